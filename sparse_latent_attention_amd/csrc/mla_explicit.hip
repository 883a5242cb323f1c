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
#include <type_traits>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// --------------------------------------------------------------------------
// Workgroup order.  Workgroups go to the eight XCDs in turn (linear id mod 8),
// and each XCD has its own L2.  `xcd_tile` deals the linear id so that the
// blocks of one head run on one XCD, one head after another: that head's
// weights (up-projection) or keys and values (attention) are then read from
// HBM about once per XCD and from its L2 after that.  Within a head, blocks
// are taken last first (the longest causal blocks start earliest).
// --------------------------------------------------------------------------
__device__ __forceinline__ void xcd_tile(int nblk, int& head, int& blk) {
    const int L = blockIdx.x;
    const int i = L >> 3;                                 // position within its XCD's queue
    head = (kHeads / 8) * (L & 7) + i / nblk;
    blk = nblk - 1 - i % nblk;
}

// --------------------------------------------------------------------------
// 1. Up-projection, a GEMM per head: D[j][t] = sum_c W[j][c] c_t[c] for the
// 256 rows j of the head's stacked weights (j < 128: W_UK[h][j], else
// W_UV[h][j - 128]) and a block of 256 positions t.  Weights are the A
// operand, latent rows the B operand.  Eight waves; wave w computes
// positions 64 (w / 2) .. +63 and rows 128 (w % 2) .. +127: 2 x 4 MFMA
// blocks of 32 x 32, 8 MFMAs against 6 16-byte LDS reads per 16 latent
// columns.  32 columns at a time are staged in LDS (two stages); each
// thread's share of a chunk comes from memory two chunks ahead, through two
// register sets, so a chunk has two chunks' worth of MFMA time to arrive.
// --------------------------------------------------------------------------
constexpr int kUpT = 256;                 // positions per workgroup
constexpr int kUpThreads = 512;
constexpr int kUpC = 32;                  // latent columns per stage
constexpr int kUpStride = 40;             // bf16 per staged row (32 + pad): conflict-free 16-byte reads
constexpr int kUpWBytes = 256 * kUpStride * 2;
constexpr int kUpXBytes = kUpT * kUpStride * 2;
constexpr int kUpStage = kUpWBytes + kUpXBytes;
constexpr int kUpChunks = kLatent / kUpC;
constexpr int kUpOutRow = 264;            // bf16 per staged output row (256 + pad)
static_assert(128 * kUpOutRow * 2 <= 2 * kUpStage, "output staging fits in the operand stages");

__global__ __launch_bounds__(kUpThreads, 1) void upproject_bf16(const __bf16* __restrict__ kv,
                                                                const __bf16* __restrict__ w_uk,
                                                                const __bf16* __restrict__ w_uv,
                                                                __bf16* __restrict__ up, int Tv, int nblk) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kUpStage];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 31, g = lane >> 5;
    int h, blk;
    xcd_tile(nblk, h, blk);
    const int t0 = blk * kUpT;

    // staging: thread tid moves columns 8 (tid % 4) .. +7 of a chunk for weight rows prow
    // (W_UK) and 128 + prow (W_UV), and for latent rows t0 + prow and t0 + 128 + prow
    const int prow = tid >> 2, pcol = 8 * (tid & 3);
    const __bf16* wk = w_uk + ((size_t)h * kNope + prow) * kLatent + pcol;
    const __bf16* wv = w_uv + ((size_t)h * kValue + prow) * kLatent + pcol;
    const __bf16* x0 = kv + (size_t)min(t0 + prow, Tv - 1) * kLatent + pcol;
    const __bf16* x1 = kv + (size_t)min(t0 + 128 + prow, Tv - 1) * kLatent + pcol;
    auto gload = [&](int c, u32x4 (&v)[4]) {
        v[0] = *reinterpret_cast<const u32x4*>(wk + c * kUpC);
        v[1] = *reinterpret_cast<const u32x4*>(wv + c * kUpC);
        v[2] = *reinterpret_cast<const u32x4*>(x0 + c * kUpC);
        v[3] = *reinterpret_cast<const u32x4*>(x1 + c * kUpC);
    };
    auto sstore = [&](int stage, const u32x4 (&v)[4]) {
        unsigned char* base = lds + stage * kUpStage + (prow * kUpStride + pcol) * 2;
        *reinterpret_cast<u32x4*>(base) = v[0];
        *reinterpret_cast<u32x4*>(base + 128 * kUpStride * 2) = v[1];
        *reinterpret_cast<u32x4*>(base + kUpWBytes) = v[2];
        *reinterpret_cast<u32x4*>(base + kUpWBytes + 128 * kUpStride * 2) = v[3];
    };

    f32x16 acc[2][4] = {};
    const int jw = 128 * (wave & 1), tw = 64 * (wave >> 1);
    auto compute = [&](int stage) {
        const __bf16* wl = reinterpret_cast<const __bf16*>(lds + stage * kUpStage) + (jw + r) * kUpStride + 8 * g;
        const __bf16* xl = reinterpret_cast<const __bf16*>(lds + stage * kUpStage + kUpWBytes) +
                           (tw + r) * kUpStride + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kUpC / 16; ++ks) {
            bf16x8 A[4], X[2];
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) A[jb] = *reinterpret_cast<const bf16x8*>(wl + 32 * jb * kUpStride + 16 * ks);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) X[tb] = *reinterpret_cast<const bf16x8*>(xl + 32 * tb * kUpStride + 16 * ks);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) acc[tb][jb] = mfma(A[jb], X[tb], acc[tb][jb]);
        }
    };
    // chunk c: staged at the top of step c - 1 from the register set it was loaded into
    // at step c - 3 (c - 2 for the first chunks); that set is then reloaded with chunk c + 2.
    // The loop body is branch-free (past the end the last chunk is loaded again and staged
    // into a stage nobody reads), so the compiler's memory-counter waits see both register
    // sets in flight and wait for the older one only.
    // The prologue leaves the sets in the loop's order (chunk 1 in set 1 issued before chunk 2
    // in set 0, and the scheduler kept from mixing the two).
    u32x4 s0[4], s1[4];
    gload(0, s0);
    sstore(0, s0);
    gload(1, s1);
    __builtin_amdgcn_sched_barrier(0);
    gload(2, s0);
    __syncthreads();
    static_assert(kUpChunks % 2 == 0, "chunks are taken in pairs");
#pragma unroll 1
    for (int c = 0; c < kUpChunks; c += 2) {
        // even step: chunk c+1 from set 1 to stage 1, set 1 <- chunk c+3; multiply stage 0
        sstore(1, s1);
        gload(min(c + 3, kUpChunks - 1), s1);
        __builtin_amdgcn_sched_barrier(0);               // the loads go out before the MFMAs
        compute(0);
        __syncthreads();
        // odd step: chunk c+2 from set 0 to stage 0, set 0 <- chunk c+4; multiply stage 1
        sstore(0, s0);
        gload(min(c + 4, kUpChunks - 1), s0);
        __builtin_amdgcn_sched_barrier(0);
        compute(1);
        __syncthreads();
    }
    // Output through LDS, half the positions at a time: lane (t = lane % 32, g) holds
    // j = 32 jb + 8 (i / 4) + 4 g + i % 4 of position 32 tb + t, written as 8-byte pieces of
    // staged rows (row stride 132 dwords: the 32 rows of one write fall in distinct banks);
    // then each position's 512 contiguous bytes go out as 32 16-byte stores, two positions
    // per store instruction.
    __bf16* ostage = reinterpret_cast<__bf16*>(lds);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        if ((wave >> 2) == half) {
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int jb = 0; jb < 4; ++jb)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        bf16x4 v;
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[tb][jb][4 * q4 + e];
                        *reinterpret_cast<bf16x4*>(ostage + (tw - 128 * half + 32 * tb + r) * kUpOutRow + jw + 32 * jb +
                                                   8 * q4 + 4 * g) = v;
                    }
        }
        __syncthreads();
#pragma unroll
        for (int pass = 0; pass < 128 / (kUpThreads / 32); ++pass) {
            const int row = pass * (kUpThreads / 32) + (tid >> 5);
            const int t = t0 + 128 * half + row;
            if (t < Tv)
                *reinterpret_cast<u32x4*>(up + ((size_t)t * kHeads + h) * (2 * kNope) + 8 * (tid & 31)) =
                    *reinterpret_cast<const u32x4*>(ostage + row * kUpOutRow + 8 * (tid & 31));
        }
        __syncthreads();
    }
}

// --------------------------------------------------------------------------
// 2. Selection bitmap, word-major: word w (positions 32w .. 32w+31) of query s
// at bm[w * S + s], so that the 128 words a tile of the attention needs are
// contiguous (its bitmap loads then take 2 cache lines rather than 128).
// Workgroup = one query: its words are built in LDS with LDS atomics
// (kBmChunk words = 262,144 positions at a time; one pass below that), then
// written to their word rows (neighbouring queries' words meet in L2; a
// workgroup of 32 queries writing whole rows was slower to build and no
// faster to read).  A listed position counts iff 0 <= t < Tv and
// t <= start_pos + s.
// --------------------------------------------------------------------------
constexpr int kBmChunk = 8192;

__global__ __launch_bounds__(256) void bitmap_build(const int32_t* __restrict__ idx, unsigned* __restrict__ bm, int S,
                                                    int k, int words, int Tv, int start_pos) {
    __shared__ unsigned w[kBmChunk];
    const int s = blockIdx.x;
    const int limit = min(Tv - 1, start_pos + s);
    const int32_t* row = idx + (size_t)s * k;
    for (int w0 = 0; w0 < words; w0 += kBmChunk) {
        const int n = min(kBmChunk, words - w0);
        for (int i = threadIdx.x; i < n; i += 256) w[i] = 0u;
        __syncthreads();
        for (int e = threadIdx.x; e < k; e += 256) {
            const int t = row[e];
            if (t < 0 || t > limit) continue;             // empty slot, past the cache or after the query
            const int wi = (t >> 5) - w0;
            if (wi >= 0 && wi < n) atomicOr(&w[wi], 1u << (t & 31));
        }
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += 256) bm[(size_t)(w0 + i) * S + s] = w[i];
        __syncthreads();
    }
}

// --------------------------------------------------------------------------
// 3. Attention.  Workgroup = (block of 128 queries, head h), dealt by
// xcd_tile; wave w owns queries 32w .. 32w+31 of the block.  Per tile of 32
// positions:
//   scores  S^T[t][q] = sum_d K[t][d] Q[q][d] (12 MFMAs, k = 192): K from LDS
//           as the A operand, the wave's queries in registers as B; lane
//           (q, g) ends up with rows t = 8 (i / 4) + 4 g + i % 4;
//   weights p = 2^(s * scale * log2(e) - m) where the bit of (q, t) is set,
//           else 0, against a fixed reference m per query: the maximum of
//           its scaled scores over the first tile's 32 positions, selected
//           or not.  The accumulator is never rescaled;
//   mix     O^T[v][q] += sum_t V^T[v][t] P^T[t][q] (8 MFMAs): the weights,
//           packed to bf16 where the scores are, are the B operand once k
//           slot 8 g' + e stands for row 4 g' + e (e < 4) or 8 + 4 g' + e - 4
//           (e >= 4) of the k-step's 16; V is staged row-major and read as
//           the A operand with the transposing LDS read (lane i of a 16-lane
//           block receives column c + i of the four rows its block's lanes
//           address, lane 4e + q addressing row r_e, columns c + 4q ..).
// A reference that is too low lets weights grow: any query whose weight sum
// exceeds 2^64 (or is not finite) makes the whole workgroup start again from
// an exact reference (a pass that computes only the masked maximum, then the
// weighted pass against it, whose largest weight is exactly 1).  So does a
// reference far above every selected score (a query with a selection and a
// weight sum below 2^-60), where weights would lose range.  Neither happens
// with scores of moderate spread; the common path has no branch.
// The weights of tile kt are computed between the score MFMAs of tile kt+1
// (a pair after each of k-steps 2..9), so the matrix cores work while the
// vector units do the exponentials; the weight sum adds the bf16 weights the
// mix multiplies.  Tiles pass
// through three LDS stages (kt: values and bitmap words, kt+1: keys, kt+2:
// being written) and two register sets (tiles kt+3 and kt+4 in flight).
// --------------------------------------------------------------------------
constexpr int kQb = 128;                  // queries per workgroup
constexpr int kKStride = 200;             // bf16 per staged key row (192 + pad)
constexpr int kVRow = 144;                // bf16 per staged value row (128 + pad: the four rows of a
                                          // transposing read fall in disjoint banks)
constexpr int kKBytes = 32 * kKStride * 2;
constexpr int kVBytes = 32 * kVRow * 2;
constexpr int kBitsBytes = kQb * 4;       // each query's bitmap word for the tile
constexpr int kStage = kKBytes + kVBytes + kBitsBytes;
constexpr int kStages = 3;
constexpr int kScAhead = 4;                // score operands read ahead of their MFMA
constexpr int kOutRow = 136;              // bf16 per staged output row (128 + pad)
static_assert(kQb * kOutRow * 2 <= kStages * kStage, "output staging fits in the tile stages");
constexpr float kSumHigh = 18446744073709551616.f;   // 2^64
constexpr float kSumLow = 8.673617379884035e-19f;    // 2^-60

__device__ __forceinline__ float pair_max(float x) {   // max over lanes l and l ^ 32
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {   // sum over lanes l and l ^ 32
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
// Transposing read of four bf16 (see the mix above).
__device__ __forceinline__ bf16x4 lds_read_tr(const unsigned char* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

struct TileRegs {
    u32x4 v[5];
    unsigned bits;
};

__global__ __launch_bounds__(256, 2) void explicit_attn_bf16(const __bf16* __restrict__ q_nope,
                                                          const __bf16* __restrict__ q_pe,
                                                          const __bf16* __restrict__ up,
                                                          const __bf16* __restrict__ pe,
                                                          const unsigned* __restrict__ bm, __bf16* __restrict__ out,
                                                          int S, int Tv, int words, int start_pos, float scale_log2,
                                                          int nqb) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kStages * kStage];
    __shared__ int rerun_vote[4];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q = lane & 31, g = lane >> 5;
    int h, qblk;
    xcd_tile(nqb, h, qblk);
    const int qb0 = qblk * kQb;
    const int qs = qb0 + 32 * wave + q;                   // this lane's query
    const bool qvalid = qs < S;
    const unsigned qmask = qvalid ? ~0u : 0u;             // a query past S selects nothing
    // positions any query of the block can see: 0 .. start_pos + last query
    const int last_q = min(qb0 + kQb, S) - 1;
    const int ntiles = (min(start_pos + last_q + 1, Tv) + 31) / 32;
    const int last = ntiles - 1;

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

    // Tile kt to registers: thread tid takes row tid / 8 and 16-byte chunks tid % 8 + 8 i of
    // its 40 (16 key-content, 8 rotary, 16 value) and query qb0 + tid % 128's bitmap word (a
    // query past S reads the last one's; its lanes ignore it).
    auto load_tile = [&](int kt, TileRegs& r) {
        r.bits = bm[(size_t)kt * S + min(qb0 + (tid & (kQb - 1)), S - 1)];
        const int row = tid >> 3, c0 = tid & 7;
        const int t = min(kt * 32 + row, Tv - 1);
        const __bf16* kvrow = up + ((size_t)t * kHeads + h) * (2 * kNope);
        const __bf16* perow = pe + (size_t)t * kRope;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int c = c0 + 8 * i;                     // 0..15 key, 16..23 rotary, 24..39 value
            const __bf16* src = c < 16 ? kvrow + 8 * c : c < 24 ? perow + 8 * (c - 16) : kvrow + kNope + 8 * (c - 24);
            r.v[i] = *reinterpret_cast<const u32x4*>(src);
        }
    };
    auto store_tile = [&](int stage, const TileRegs& r) {
        unsigned char* kb = lds + stage * kStage;
        const int row = tid >> 3, c0 = tid & 7;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int c = c0 + 8 * i;
            unsigned char* dst = c < 24 ? kb + (row * kKStride + 8 * c) * 2
                                        : kb + kKBytes + (row * kVRow + 8 * (c - 24)) * 2;
            *reinterpret_cast<u32x4*>(dst) = r.v[i];
        }
        reinterpret_cast<unsigned*>(kb + kKBytes + kVBytes)[tid & (kQb - 1)] = r.bits;   // twice, same value
    };
    // scores: A = K[t][16 ks + 8 g' .. +7] for t = lane % 32
    auto scores = [&](int stage) {
        f32x16 sc = {};
        const __bf16* krow = reinterpret_cast<const __bf16*>(lds + stage * kStage) + q * kKStride + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 12; ++ks) sc = mfma(*reinterpret_cast<const bf16x8*>(krow + 16 * ks), qf[ks], sc);
        return sc;
    };
    // transposing-read addresses: lane (v = 32 vb + lane % 32, g) of a 16-lane block
    // addresses row 4 g + (lane % 16) / 4 (+ 8 for the second half of a k-step, + 16 kc)
    // and columns 32 vb + 16 ((lane / 16) % 2) + 4 (lane % 4) ..
    const int tr_off = ((4 * g + ((lane & 15) >> 2)) * kVRow + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

    f32x16 acc[4];
    float l_run, m_ref, m_max;
    unsigned sel_or;

    // One pass over the block's tiles.  kMaxOnly: the masked maximum of the scaled scores
    // (m_max); otherwise the weights against m_ref (taken from the first tile if
    // kFirstRef), their sum (l_run) and the mix (acc).
    auto pass = [&](auto max_only, auto first_ref) {
        constexpr bool kMaxOnly = decltype(max_only)::value;
        constexpr bool kFirstRef = decltype(first_ref)::value;
        f32x16 s_cur;
        // Step kt: tile kt+2 from its register set to LDS, that set <- tile kt+4, then the
        // scores of tile kt+1 with the weights of tile kt between their MFMAs (one pair of
        // weights after each of k-steps 2..9, so that the exponentials issue while an MFMA
        // runs, once the chain's first operand reads are under way) and the mix of tile kt
        // between them too, as soon as its weights are complete: its MFMAs are independent of
        // the chain's and fill the chain's dependency gaps.  Operands are read from LDS
        // several MFMAs ahead.  Branch-free, so
        // that the compiler's memory-counter waits see both register sets in flight: past
        // the last tile the last one is loaded and staged again into a stage nobody reads,
        // and the scores beyond it are dropped.
        auto step = [&](int kt, TileRegs& set) {
            store_tile((kt + 2) % kStages, set);
            load_tile(min(kt + 4, last), set);
            __builtin_amdgcn_sched_barrier(0);           // the loads go out before the MFMAs
            const unsigned char* kb = lds + (kt % kStages) * kStage;
            const unsigned word = reinterpret_cast<const unsigned*>(kb + kKBytes + kVBytes)[32 * wave + q];
            const unsigned bits = (word >> (4 * g)) & qmask;
            // Weights in bf16 pairs (elements i, i+1: positions t, t+1): both converted at
            // once, then the unselected half zeroed with a byte mask, and the pair's sum
            // added to l_run by one dot product with (1, 1), so that l_run adds exactly the
            // weights the mix multiplies.  The masks come from the byte permute's
            // sign-replicating selectors (8: bit 15 of its second source, 9: bit 31; 10, 11:
            // the same of its first): sh[b] holds the bits moved up so that position b sits
            // at bit 15 and position b + 16 at bit 31.
            unsigned sh[8];
#pragma unroll
            for (int b = 0; b < 8; ++b) sh[b] = bits << (15 - ((b & 3) + 8 * (b >> 2)));
            u32x4v pw[2];
            float psum = 0.f;
            const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
            auto weights = [&](int i) {                   // elements i, i + 1 (i even)
                if constexpr (kMaxOnly) {
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int t = 8 * (i >> 2) + (i & 3) + e;
                        m_max = (bits >> t) & 1u ? fmaxf(m_max, s_cur[i + e] * scale_log2) : m_max;
                    }
                } else {
                    const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[i], scale_log2, -m_ref));
                    const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[i + 1], scale_log2, -m_ref));
                    const bf16x2 pe2 = {(__bf16)e0, (__bf16)e1};
                    // positions t = 8 (i / 4) + i % 4 and t + 1; below 16 they sit at bit 15
                    // of sh[b], sh[b + 1], from 16 on at bit 31 of them
                    const int b = (i & 3) + 4 * ((i >> 2) & 1);
                    const unsigned sel = i < 8 ? 0x0A0A0808u : 0x0B0B0909u;
                    const unsigned pm =
                        __builtin_bit_cast(unsigned, pe2) & __builtin_amdgcn_perm(sh[b + 1], sh[b], sel);
                    psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pm), ones, psum, false);
                    pw[i >> 3][(i >> 1) & 3] = pm;
                }
            };
            // scores of tile kt+1: A = K[t][16 ks + 8 g' .. +7] for t = lane % 32
            const __bf16* krow =
                reinterpret_cast<const __bf16*>(lds + ((kt + 1) % kStages) * kStage) + q * kKStride + 8 * g;
            bf16x8 pre[kScAhead];
#pragma unroll
            for (int d = 0; d < kScAhead; ++d) pre[d] = *reinterpret_cast<const bf16x8*>(krow + 16 * d);
            f32x16 s_next = {};
            // mix m = 4 kc + vb: acc[vb] += V^T[32 vb ..][16 kc ..] P^T, interleaved with the
            // chain: the weights of elements 0..7 (pb[0]) are done after k-step 5, those of
            // 8..15 after k-step 9; mix MFMAs m = 0..3 follow k-steps 6..9 and m = 4..7 two each
            // follow k-steps 10 and 11, in the gaps of the chain's dependent MFMAs.  Each
            // accumulator still takes its two MFMAs in the order kc = 0, 1.
            const unsigned char* vb0 = kb + kKBytes + tr_off;
            auto vread = [&](int m) {
                const unsigned char* a0 = vb0 + (16 * (m >> 2) * kVRow + 32 * (m & 3)) * 2;
                return cat(lds_read_tr(a0), lds_read_tr(a0 + 8 * kVRow * 2));
            };
            bf16x8 va[8];
            // Raised wave priority for this phase: with two workgroups per CU each SIMD runs two
            // waves, and the one in its score chain then issues ahead of one storing a tile or
            // waiting at the barrier.
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int ks = 0; ks < 12; ++ks) {
                const bf16x8 av = pre[ks % kScAhead];
                if (ks + kScAhead < 12) pre[ks % kScAhead] = *reinterpret_cast<const bf16x8*>(krow + 16 * (ks + kScAhead));
                s_next = mfma(av, qf[ks], s_next);
                if (ks >= 2 && ks < 10) weights(2 * (ks - 2));
                if constexpr (!kMaxOnly) {
                    // mix operands: m = 0..3 read at k-steps 3..6, m = 4..7 at 7..10
                    if (ks >= 3 && ks < 11) va[ks - 3] = vread(ks - 3);
                    // mix MFMAs: m = 0..3 after k-steps 6..9 (pb[0] complete after k-step 5),
                    // m = 4..7 after k-steps 10, 10, 11, 11 (pb[1] complete after k-step 9)
                    if (ks >= 6 && ks < 10) {
                        const int m = ks - 6;
                        const bf16x8 pb0 = __builtin_bit_cast(bf16x8, pw[0]);
                        acc[m] = mfma(va[m], pb0, acc[m]);
                    }
                    if (ks >= 10) {
                        const bf16x8 pb1 = __builtin_bit_cast(bf16x8, pw[1]);
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const int m = 4 + 2 * (ks - 10) + u;
                            acc[m & 3] = mfma(va[m], pb1, acc[m & 3]);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_s_setprio(0);
            if constexpr (!kMaxOnly) {
                sel_or |= bits;
                l_run += psum;
            }
            s_cur = s_next;
            __syncthreads();                              // stage kt free; stage kt+2 complete
        };
        // The prologue leaves tiles 2 and 3 in flight in the loop's order (set ra's loads
        // first, the scheduler kept from mixing the two sets).
        TileRegs ra, rb;                                  // tiles 2j and 2j+1
        load_tile(0, ra);
        load_tile(min(1, last), rb);
        store_tile(0, ra);
        store_tile(1, rb);
        load_tile(min(2, last), ra);
        __builtin_amdgcn_sched_barrier(0);
        load_tile(min(3, last), rb);
        __syncthreads();
        s_cur = scores(0);
        if constexpr (kFirstRef) {
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s_cur[i] * scale_log2);
            m_ref = pair_max(mx);
        }
        int kt = 0;
        for (; kt + 1 < ntiles; kt += 2) {
            step(kt, ra);
            step(kt + 1, rb);
        }
        if (kt < ntiles) step(kt, ra);
    };
    auto clear = [&]() {
#pragma unroll
        for (int vb = 0; vb < 4; ++vb) acc[vb] = f32x16{};
        l_run = 0.f;
        sel_or = 0u;
    };

    clear();
    pass(std::false_type{}, std::true_type{});
    float lt = pair_sum(l_run);
    const bool has_sel = pair_sum(sel_or != 0u ? 1.f : 0.f) > 0.f;
    const bool bad = !(lt <= kSumHigh) || (has_sel && lt < kSumLow);
    const bool wave_bad = __builtin_amdgcn_ballot_w64(bad) != 0;   // every lane takes part
    if (lane == 0) rerun_vote[wave] = wave_bad;
    __syncthreads();
    if (rerun_vote[0] | rerun_vote[1] | rerun_vote[2] | rerun_vote[3]) {
        m_max = -INFINITY;
        pass(std::true_type{}, std::false_type{});
        const float mx = pair_max(m_max);
        m_ref = mx == -INFINITY ? 0.f : mx;               // no selection: every weight is 0 anyway
        clear();
        pass(std::false_type{}, std::false_type{});
        lt = pair_sum(l_run);
    }

    // Normalise and store through LDS: lane (q, g) holds v = 32 vb + 8 (i / 4) + 4 g + i % 4
    // of query 32 wave + q, written as 8-byte pieces of staged rows (row stride 68 dwords: the
    // 32 rows of one write fall in distinct banks); then each query's 256 contiguous bytes go
    // out as 16 16-byte stores, four queries per store instruction.  Every wave is past the
    // last barrier of its passes, so the stages are free.
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    __bf16* ostage = reinterpret_cast<__bf16*>(lds);
#pragma unroll
    for (int vb = 0; vb < 4; ++vb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[vb][4 * gq + e] * inv);
            *reinterpret_cast<bf16x4*>(ostage + (32 * wave + q) * kOutRow + 32 * vb + 8 * gq + 4 * g) = v;
        }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < kQb / 16; ++pass) {
        const int row = pass * 16 + (tid >> 4);
        if (qb0 + row < S)
            *reinterpret_cast<u32x4*>(out + ((size_t)(qb0 + row) * kHeads + h) * kValue + 8 * (tid & 15)) =
                *reinterpret_cast<const u32x4*>(ostage + row * kOutRow + 8 * (tid & 15));
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
    const int nblk = (p.Tv + kUpT - 1) / kUpT;
    hipLaunchKernelGGL(upproject_bf16, dim3((unsigned)nblk * kHeads), dim3(kUpThreads), 0, s,
                       static_cast<const __bf16*>(kv), static_cast<const __bf16*>(w_uk),
                       static_cast<const __bf16*>(w_uv), up, p.Tv, nblk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bitmap_build, dim3((unsigned)S), dim3(256), 0, s, idx, bm, S, k, p.words, p.Tv, start_pos);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int nqb = (S + kQb - 1) / kQb;
    hipLaunchKernelGGL(explicit_attn_bf16, dim3((unsigned)nqb * kHeads), dim3(256), 0, s,
                       static_cast<const __bf16*>(q_nope), static_cast<const __bf16*>(q_pe), up,
                       static_cast<const __bf16*>(pe), bm, static_cast<__bf16*>(out), S, p.Tv, p.words, start_pos,
                       scale_log2, nqb);
    return hipGetLastError();
}

}  // namespace mla
