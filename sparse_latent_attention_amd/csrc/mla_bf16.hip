// bf16 kernels for gfx950 (CDNA4): W_UK absorption, sparse latent attention,
// split merge + W_UV absorption.  All matrix products run on bf16 MFMA with
// float32 accumulation.
//
// MFMA operand layouts used below (64-lane wavefront, l = lane id):
//   v_mfma_f32_16x16x32_bf16: A[m][k] from lane (m + 16*(k/8)), element k%8;
//     B[k][n] from lane (n + 16*(k/8)), element k%8; D[m][n] in lane
//     (n + 16*(m/4)), element m%4.
//   v_mfma_f32_32x32x16_bf16: A[m][k] from lane (m + 32*(k/8)), element k%8;
//     B[k][n] from lane (n + 32*(k/8)), element k%8; D[m][n] in lane
//     (n + 32*((m/4)%2)), element 4*(m/8) + m%4.
// Any permutation of k applied to both operands leaves the product unchanged;
// the attention kernel uses that to match the transposing LDS read below.
//
// ds_read_b64_tr_b16 (transposing LDS read): within each 16-lane block, lane
// i receives element e (e = 0..3) from the 8-byte chunk addressed by lane
// 4e + i/4, element i%4.  If lane 4e + q of a block addresses row r_e,
// columns c + 4q .. c + 4q + 3 of a row-major bf16 matrix, lane i of the
// block receives column c + i of rows r_0 .. r_3: a column-major MFMA operand
// read from row-major storage.
#include <hip/hip_ext.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 to_bf16x4(float a, float b, float c, float d) {
    bf16x4 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    r[2] = (__bf16)c;
    r[3] = (__bf16)d;
    return r;
}

// Score-chain MFMAs with the accumulator in ordinary VGPRs.  The mix
// accumulator takes all 256 accumulation registers, so the compiler (which
// picks one MFMA register form per kernel) would otherwise shuttle the score
// tile through them.  Chained MFMAs that read the previous result as their
// accumulator input (exact overlap) need no wait states.  The compiler does
// not see these as MFMAs, so the last one of a chain carries the wait states
// an MFMA result needs before any other instruction may read it; the result
// is not available to the compiler before that.
__device__ __forceinline__ void mfma32_v_first(f32x16& d, bf16x8 a, bf16x8 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_v(f32x16& d, bf16x8 a, bf16x8 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// The final MFMA writes a separate register tuple, so that no copy of the
// chain's accumulator can be placed before the chain has finished.
__device__ __forceinline__ void mfma32_v_last(f32x16& out, const f32x16& d, bf16x8 a, bf16x8 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "=&v"(out) : "v"(a), "v"(b), "v"(d));
}

// Transposing read of four bf16 (see the header comment).
__device__ __forceinline__ bf16x4 lds_read_tr(const lds_u8* p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// A raw buffer load whose offset is >= its descriptor's size returns zeros
// without touching memory; kOutOfRange is such an offset for every buffer
// these kernels describe (<= 2 GiB; see make_desc).
constexpr unsigned kOutOfRange = 0x80000000u;

// Combine the values of lanes l and l ^ 32 (v_permlane32_swap exchanges the
// upper half of one register with the lower half of the other: swapping a
// value with itself leaves, in the two results, the lower and the upper half
// of the wave broadcast to both halves).  Needs no address register, unlike
// a shuffle through ds_bpermute.
__device__ __forceinline__ float pair_max(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}
// This lane's index within its wave, from the execution mask (no register
// needs to hold it: after a long loop that uses every register, the compiler
// would otherwise reload a spilled thread index from scratch memory).
__device__ __forceinline__ int lane_id() {
    return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Layout of the absorbed queries in the workspace; element c (0..575: 512
// latent, then 64 rotary) of head h of query row r sits at
//   ((r*4 + h/32)*36 + c/16)*512 + (h%32)*16 + c%16     (operand image), or
//   (r*128 + h)*576 + c                                 (row-major).
// The operand image suits the attention waves' score operands: the 16-byte
// operand loads of one wave and k-step read one contiguous 1 KiB run, but the
// absorption writes it in 32-byte pieces.  Row-major, the absorption writes
// whole lines and the operand loads read 32 bytes from each of 32 rows.  Few
// query rows (decode) take the image: there the absorption's stores are a few
// MB and the attention's prologue waits for its queries.  Many rows (a prefill
// chunk) take row-major: there the absorbed queries are hundreds of MB written
// once, and each workgroup's query loads are a small part of its work.
constexpr int kQRowMajorMinRows = 512;
__device__ __forceinline__ size_t q_off(int r, int h, int c, bool rowmajor) {
    return rowmajor ? ((size_t)r * kHeads + h) * kQRow + c
                    : (((size_t)r * 4 + (h >> 5)) * 36 + (c >> 4)) * 512 + (size_t)((h & 31) * 16) + (c & 15);
}

// --------------------------------------------------------------------------
// Step 1: q_c[r, h, :] = q_nope[r, h, :] . W_UK[h]  (and append q_pe)
//
// Per head this is a [R x 128] . [128 x 512] product, computed transposed,
// q_c^T = W_UK[h]^T . q_nope^T: the weight is the A operand (its columns c
// become MFMA rows) and each lane's output holds four consecutive c of one
// query row.  Workgroup = (head, quarter of c, group of 32-row query blocks).
// The weight slice [128 d x 128 c] is staged in LDS with 16-byte loads and
// read back transposed; wave w keeps the fragments of its 32 columns in
// registers for every query block it visits.  A query block (32 rows x 128 d)
// is the B operand of all four waves: the workgroup loads it once (32 bytes
// per thread), stages it in LDS and each wave reads its fragments from there.
// The first two blocks are loaded together with the weight (one memory round
// trip), and each output block goes through LDS so that every row segment
// (128 c = 256 bytes) is written by 16 consecutive lanes.
// --------------------------------------------------------------------------
constexpr int kWRow = 320;   // bytes per staged W_UK row (128 bf16 + pad)
constexpr int kQcRow = 272;  // bytes per staged output row (128 bf16 + pad)

constexpr int kQnRow = 272;  // bytes per staged query row (128 bf16 + pad)

// LDS one absorb unit uses: the weight slice, one output block, two query blocks
constexpr int kAbsorbLds = kNope * kWRow + 32 * kQcRow + 2 * 32 * kQnRow;

// One unit = (head h, quarter cq of the 512 latent columns), for query blocks
// rb_first, rb_first + rb_step, ...; `lds` holds kAbsorbLds bytes.  Every
// thread of the workgroup calls it.
template <bool kRowMajor>
__device__ __forceinline__ void absorb_unit(const __bf16* __restrict__ q_nope,
                                            const __bf16* __restrict__ q_pe,
                                            const __bf16* __restrict__ w_uk,
                                            __bf16* __restrict__ q_out, int R, int unit,
                                            int rb_first, int r_groups, unsigned char* lds) {
    unsigned char* wbuf = lds;
    unsigned char* obuf = lds + kNope * kWRow;
    unsigned char* qbuf[2] = {obuf + 32 * kQcRow, obuf + 32 * kQcRow + 32 * kQnRow};
    const int h = unit >> 2;
    const int cq = unit & 3;
    const int tid = threadIdx.x;
    const int wave = wave_id();
    const int lane = tid & 63;
    const int half = lane >> 5;

    // One 32-row query block: thread t fetches 32 bytes, row t/8, columns
    // d = 16*(t%8) .. +15 (rows past R read as zeros), and stages them in LDS.
    // The column quarter cq = 0 also copies the block's q_pe rows (thread t:
    // row t/8, 16-byte chunk t%8), loaded here with the block so that the copy
    // adds no memory round trip after the multiply.
    auto load_q = [&](int rb, u32x4 (&p)[3]) {
        const int r = rb * 32 + (tid >> 3);
        const bool rv = r < R;
        const __bf16* qn = q_nope + ((size_t)(rv ? r : 0) * kHeads + h) * kNope + 16 * (tid & 7);
        p[0] = rv ? *reinterpret_cast<const u32x4*>(qn) : u32x4{};
        p[1] = rv ? *reinterpret_cast<const u32x4*>(qn + 8) : u32x4{};
        p[2] = rv && cq == 0 ? *reinterpret_cast<const u32x4*>(q_pe + ((size_t)r * kHeads + h) * kRope + 8 * (tid & 7))
                             : u32x4{};
    };
    auto stage_q = [&](const u32x4 (&p)[3], unsigned char* qb, u32x4& pe) {
        unsigned char* dst = qb + (tid >> 3) * kQnRow + 32 * (tid & 7);
        *reinterpret_cast<u32x4*>(dst) = p[0];
        *reinterpret_cast<u32x4*>(dst + 16) = p[1];
        pe = p[2];
    };
    // B fragments of a staged block: q_nope[r][h][16ks + 8half .. +7], r = lane % 32
    auto frags_q = [&](const unsigned char* qb, bf16x8 (&b)[8]) {
        const unsigned char* src = qb + (lane & 31) * kQnRow + 16 * half;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) b[ks] = *reinterpret_cast<const bf16x8*>(src + 32 * ks);
    };
    const int blocks = (R + 31) / 32;
    bf16x8 b0[8], b1[8];
    u32x4 p0[3], p1[3];
    u32x4 pe0 = {}, pe1 = {};          // q_pe chunks of the blocks in b0 and b1
    load_q(rb_first, p0);
    if (rb_first + r_groups < blocks) load_q(rb_first + r_groups, p1);

    {
        // 128 rows d x 16 chunks of 8 columns; 8 chunks per thread
        const __bf16* src = w_uk + (size_t)h * kNope * kLatent + cq * 128;
        u32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = tid + 256 * i;
            v[i] = *reinterpret_cast<const u32x4*>(src + (size_t)(e >> 4) * kLatent + 8 * (e & 15));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = tid + 256 * i;
            *reinterpret_cast<u32x4*>(wbuf + (e >> 4) * kWRow + 16 * (e & 15)) = v[i];
        }
    }
    stage_q(p0, qbuf[0], pe0);
    if (rb_first + r_groups < blocks) stage_q(p1, qbuf[1], pe1);
    __syncthreads();
    frags_q(qbuf[0], b0);
    if (rb_first + r_groups < blocks) frags_q(qbuf[1], b1);

    // A fragments: W_UK[h][d][c] for c = 32*wave + lane%32 (within the quarter),
    // d = 16*ks + 8*half + e (e = 0..7) via two transposing reads.
    bf16x8 a[8];
    {
        const int blk = lane >> 4, e4 = (lane & 15) >> 2, q = lane & 3;
        const lds_u8* base = (const lds_u8*)wbuf + (8 * (blk >> 1) + e4) * kWRow +
                             (32 * wave + 16 * (blk & 1) + 4 * q) * 2;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            a[ks] = cat(lds_read_tr(base + 16 * ks * kWRow), lds_read_tr(base + (16 * ks + 4) * kWRow));
    }

    // `last`: no later block of this workgroup reuses the staging
    auto process = [&](int rb, const bf16x8 (&b)[8], const u32x4& pe, bool last) {
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) acc = mfma32(a[ks], b[ks], acc);
        // lane holds c = 32*wave + 8g + 4*half .. +3 of row lane % 32
        unsigned char* mine = obuf + (lane & 31) * kQcRow + (32 * wave + 4 * half) * 2;
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *reinterpret_cast<bf16x4*>(mine + 16 * g) =
                to_bf16x4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
        __syncthreads();
        // 32 rows x 16 chunks of 16 bytes: two chunks per thread
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = tid + 256 * i;
            const int rr = rb * 32 + (e >> 4);
            if (rr < R)
                *reinterpret_cast<u32x4*>(q_out + q_off(rr, h, cq * 128 + 8 * (e & 15), kRowMajor)) =
                    *reinterpret_cast<const u32x4*>(obuf + (e >> 4) * kQcRow + 16 * (e & 15));
        }
        if (cq == 0) {
            // q_pe rows of this block: 32 rows x 8 chunks of 16 bytes = one per thread.
            const int rr = rb * 32 + (tid >> 3);
            if (rr < R) *reinterpret_cast<u32x4*>(q_out + q_off(rr, h, kLatent + 8 * (tid & 7), kRowMajor)) = pe;
        }
        if (!last) __syncthreads();       // obuf reused by the next block
    };
    // Two query blocks in flight: while one is multiplied, the next but one
    // loads; it is staged once every wave has its fragments of the block
    // before (process ends with a barrier) and read back after the barrier
    // below.
    for (int rb = rb_first; rb < blocks; rb += 2 * r_groups) {
        const bool more0 = rb + 2 * r_groups < blocks;
        const bool has1 = rb + r_groups < blocks;
        const bool more1 = rb + 3 * r_groups < blocks;
        if (more0) load_q(rb + 2 * r_groups, p0);
        process(rb, b0, pe0, !has1);
        if (more0) stage_q(p0, qbuf[0], pe0);
        if (has1) {
            if (more1) load_q(rb + 3 * r_groups, p1);
            process(rb + r_groups, b1, pe1, !more0);
            if (more1) stage_q(p1, qbuf[1], pe1);
        }
        if (more0) {
            __syncthreads();              // staged blocks visible
            frags_q(qbuf[0], b0);
            if (more1) frags_q(qbuf[1], b1);
        }
    }
}

// kRowMajor: write the absorbed queries row-major (R >= kQRowMajorMinRows), else the operand image.
template <bool kRowMajor>
__global__ __launch_bounds__(256) void absorb_q_bf16(const __bf16* __restrict__ q_nope,
                                                     const __bf16* __restrict__ q_pe,
                                                     const __bf16* __restrict__ w_uk,
                                                     __bf16* __restrict__ q_out, int R,
                                                     int r_groups, int* stats) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kAbsorbLds];
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 2) stats[threadIdx.x] = 0;   // the call's diagnostics
    // Workgroups are dealt to the eight XCDs in turn (id % 8).  XCD x takes
    // heads 16x .. 16x+15 with all four column quarters, so a head's queries
    // come from memory once per launch (the other quarters hit that XCD's L2)
    // and the 32-byte output pieces of neighbouring heads, which share cache
    // lines, are merged in one L2 before they are written back.
    const int b = blockIdx.x, j = b >> 3;
    absorb_unit<kRowMajor>(q_nope, q_pe, w_uk, q_out, R, (16 * (b & 7) + (j >> 2)) * 4 + (j & 3), blockIdx.y,
                r_groups, lds);
}

// --------------------------------------------------------------------------
// Steps 2-4: sparse attention over the selected latent rows.
//
// Workgroup = (query row r, split of its index list): four waves, wave w owns
// heads 32w .. 32w+31 and every selected row of the split, so no wave waits on
// another except to share the row tiles.  Selected rows are gathered 32 at a
// time straight into LDS (buffer loads with an LDS destination, so the data
// never occupies registers) through four tile buffers: three tiles are in
// flight while one is consumed, and one barrier per tile hands a buffer from
// readers to the next gather.  Per tile and wave:
//   scores   S^T[j][h] = sum_c row_j[c] Q[h][c] (v_mfma 32x32x16, Q in
//            registers as the B operand); each lane ends up owning one head h
//            and sixteen rows j;
//   softmax  per lane, in the log2 domain, against a reference m taken from
//            the head's first tile with a selected row: p = 2^(s - m).  The
//            accumulator is never rescaled (which keeps it in the
//            accumulation registers).  If a lane's probabilities in one tile
//            sum past 2^64 (a later score beat m by about 60), which no
//            realistic attention does, the workgroup runs the split again
//            with each head's largest score as m (kRerunSum);
//   mix      O~^T[c][h] += sum_j V^T[c][j] P^T[j][h] over all 512 columns c of
//            the wave's own heads (v_mfma 32x32x16).  The probabilities, packed
//            to bf16 where the score accumulator left them, already form the
//            B operand of the mix, provided MFMA k slot 4t + e of lane half g
//            is row 16kc + 8t + 4g + e; V^T comes from the row-major tile
//            through the transposing LDS read with the same slot order.  So P
//            never leaves registers and no wave waits for another between the
//            softmax and the mix.
// LDS tile layout: latent rows at 1024-byte stride with 16-byte chunk q of
// row j stored at chunk q ^ swz(j); rotary rows in four 8-row blocks (1152-byte
// stride) with chunk c of block row j' at c ^ j'.  Both the score reads and the
// transposing reads then touch each bank once per pass.
// Empty or out-of-range slots load with an out-of-range buffer offset (no
// memory access) and are masked to -inf before the softmax.
// --------------------------------------------------------------------------
constexpr int kRows = kTileRows;             // rows per tile
constexpr int kBufs = 4;                     // tile buffers
constexpr int kLatBytes = kRows * 1024;
constexpr int kPeBlock = 1152;               // 8 rotary rows (1 KiB) + 128-byte pad
constexpr int kBufBytes = kLatBytes + 4 * kPeBlock;

// Workgroup barrier after this wave's LDS writes have completed.  Written as
// assembly with a memory clobber so that the compiler keeps LDS accesses on
// their side of it; global loads in flight (the gathers) are not waited for.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void barrier_only() {
    asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ int lat_swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
#define MLA_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

// 16-byte-per-lane buffer load straight into LDS: lane l's 16 bytes land at
// LDS byte address lds_addr + 16*l (lds_addr must be wave-uniform); an offset
// past the buffer's size reads zeros.  Written as inline assembly so that the
// compiler does not order the kernel's LDS reads behind every gather in flight
// (it cannot tell the tile buffers apart); the kernel orders them itself with
// explicit vmcnt waits and barriers.  No register receives data, and M0 is
// restored before the block ends.
__device__ __forceinline__ void load_lds16(u32x4 rsrc, unsigned lds_addr, unsigned voff) {
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_addr), "v"(voff), "s"(rsrc)
        : "memory");
}

// Four such loads into the LDS rows lds_addr, +1 KiB, +2 KiB, +3 KiB with a
// single M0 value: the instruction offset (0, 1024, 2048, 3072) moves both the
// LDS destination and the memory address, so each memory offset passed in is
// its true offset + 3072 - 1024*u, against a descriptor whose base sits 3 KiB
// before the data (see make_desc_x4).  Rewriting M0 before every load would
// hold each load until the previous one has landed, which caps a wave at one
// load in flight; this way four are.
constexpr unsigned kX4Bias = 3072u;
__device__ __forceinline__ void load_lds16_x4(u32x4 rsrc, unsigned lds_addr, unsigned v0, unsigned v1,
                                              unsigned v2, unsigned v3) {
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %6, 0 offen lds\n\t"
        "buffer_load_dwordx4 %3, %6, 0 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %4, %6, 0 offen offset:2048 lds\n\t"
        "buffer_load_dwordx4 %5, %6, 0 offen offset:3072 lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_addr), "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(rsrc)
        : "memory");
}
// Offset for lane data at true offset `off` of load u of a group (or out of range).
__device__ __forceinline__ unsigned x4_off(bool ok, unsigned off, int u) {
    return ok ? off + kX4Bias - 1024u * (unsigned)u : kOutOfRange;
}

// Raw buffer descriptor (stride 0) over `bytes` bytes at `base`.
__device__ __forceinline__ u32x4 make_desc(const void* base, unsigned bytes) {
    const unsigned long long b = reinterpret_cast<unsigned long long>(base);
    return u32x4{(unsigned)b, (unsigned)(b >> 32) & 0xFFFFu, bytes, 0x00020000u};
}
// Descriptor for load_lds16_x4 over `bytes` bytes at `base`: it starts kX4Bias
// bytes early and covers them too (the loads never touch that prefix).
__device__ __forceinline__ u32x4 make_desc_x4(const void* base, unsigned bytes) {
    const unsigned long long b = reinterpret_cast<unsigned long long>(base) - kX4Bias;
    return u32x4{(unsigned)b, (unsigned)(b >> 32) & 0xFFFFu, bytes + kX4Bias, 0x00020000u};
}

// Everything one workgroup needs to process one (query row, split).
struct SplitCtx {
    const AttnArgs* a;
    unsigned char* tiles;        // kBufs tile buffers in LDS (generic pointer to LDS)
    int* sidx;                   // the split's index list in LDS (-1 past its end)
    const int32_t* idx_src;      // the split's index list in global memory
    int nslots;                  // its length
    const __bf16* qrow;          // this lane's score operands: k-step ks at qrow + 512*ks (image) or 16*ks
    u32x4 kv_desc, pe_desc;
    int r, split, ntiles, limit, T, wave, lane;
};

// Score operands read ahead of their MFMA: LDS reads only reach full
// bandwidth with many in flight per wave, and every wave streams a whole tile
// through the score chain.
#ifndef MLA_SC_DEPTH
#define MLA_SC_DEPTH 6
#endif
constexpr int kScDepth = MLA_SC_DEPTH;
// V^T operands of the mix read ahead of their MFMA.  The hand-over barrier
// sits before the last four MFMAs of a mix, and every read of the tile must
// be issued ahead of it (the barrier then also certifies that they landed).
#ifndef MLA_MIX_DEPTH
#define MLA_MIX_DEPTH 4
#endif
constexpr int kMixDepth = MLA_MIX_DEPTH;
static_assert(kMixDepth >= 3 && kMixDepth <= 8, "mix read-ahead out of range");

// While no lane's probabilities in one tile sum past this (no scaled score
// beat its head's reference by more than about 60 in log2 units), no
// probability, partial sum of at most 2048 of them, or mix of them with
// latent values comes near the float range; probabilities far below the
// reference underflow to 0 exactly where they are negligible against the
// reference's own weight of 1.  A split whose sum does pass it is run again:
// first a pass that only finds each head's largest score, then the full pass
// with that as the reference, so that every probability is at most 1.
constexpr float kRerunSum = 18446744073709551616.f;   // 2^64

// One pass over the split's tiles.  Software pipeline, per iteration t: the
// score MFMAs of tile t+1 run with the softmax of tile t and the gathers of
// tile t+3 interleaved between them (VALU and memory instructions issue while
// an MFMA executes), then the mix MFMAs of tile t, with the hand-over to the
// next iteration (own gathers of tile t+2 landed, then a barrier) before its
// last four MFMAs.
// The reference of each head is the (scaled) maximum of its first tile with
// a selected row, or, with `preset`, the value m_ref holds on entry.  The
// accumulator is never rescaled; `beaten` reports a tile whose probabilities
// passed kRerunSum (the pass's result is then to be discarded).
// kMaxOnly: the same tile pipeline with no exponentials and no mix; on
// return m_ref holds each head's largest scaled score over the selected rows.
template <bool kMaxOnly, bool kRowMajor>
__device__ __forceinline__ void attn_pass(const SplitCtx& c, float& m_ref, f32x16 (&acc)[16],
                                          float& l_run, bool& beaten, bool preset) {
    const int lane = c.lane;
    beaten = false;
    // A slot is selected iff 0 <= p < lim (p < T and, for prefill, p <= limit).
    const unsigned lim = min((unsigned)c.T, (unsigned)c.limit + 1u);
    // Query fragments (B operands): head 32*wave + lane%32, columns
    // 16*ks + 8*(lane/32) .. +7.  Retiring their loads here leaves vmcnt
    // counting the gathers only inside the tile loop.
    // Prologue: the split's index list and the query fragments are in flight
    // together; tile 0 follows once the list is in LDS, and tiles 1 and 2 go
    // out during tile 0's score chain.
    constexpr int kIdxPerThread = kMaxSlotsPerSplit / 256;
    int iv[kIdxPerThread];
#pragma unroll
    for (int u = 0; u < kIdxPerThread; ++u) {
        const int i = (int)threadIdx.x + 256 * u;
        iv[u] = i < c.nslots ? c.idx_src[i] : -1;
    }
    bf16x8 qf[36];
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(c.qrow + (kRowMajor ? 16 : 512) * ks);
    // The split's last selected slot: tiles past it hold no selected row (a
    // causal prefill query early in its chunk leaves most of its list empty)
    // and are not processed.
    // For this wave (slots threadIdx.x + 256 u): the highest u with a selected
    // slot in some lane, and there the highest such lane, from one ballot per
    // u (shuffles would put a chain of LDS round trips before the list's store).
    int last_sel = -1;
#pragma unroll
    for (int u = kIdxPerThread - 1; u >= 0; --u) {
        const int i = (int)threadIdx.x + 256 * u;
        const unsigned long long m = __builtin_amdgcn_ballot_w64(i < c.nslots && (unsigned)iv[u] < lim);
        if (last_sel < 0 && m != 0ull) last_sel = 256 * u + 64 * c.wave + (63 - __builtin_clzll(m));
    }
    if (lane == 0) c.sidx[kMaxSlotsPerSplit + c.wave] = last_sel;
#pragma unroll
    for (int u = 0; u < kIdxPerThread; ++u) {
        const int i = (int)threadIdx.x + 256 * u;
        if (i < c.ntiles * kRows) c.sidx[i] = iv[u];
    }
    barrier_lds();
    const int* wave_last = c.sidx + kMaxSlotsPerSplit;
    const int ntiles = (max(max(wave_last[0], wave_last[1]), max(wave_last[2], wave_last[3])) + kRows) / kRows;
    if constexpr (!kMaxOnly) {
#pragma unroll
        for (int cb = 0; cb < 16; ++cb) acc[cb] = f32x16{};
    }
    l_run = kMaxOnly ? -INFINITY : 0.f;  // max-only passes keep their running maximum here
    if (ntiles == 0) {                   // nothing selected: an empty partial
        __builtin_amdgcn_s_waitcnt(0);   // no load may land after the workgroup ends
        if constexpr (kMaxOnly) m_ref = -INFINITY;
        return;
    }

    // Per-lane LDS offsets, relative to a tile buffer.  Buffer offsets are
    // multiples of 512 bytes, so XOR-ing a compile-time constant into bits 5..7
    // of an offset commutes with adding the buffer offset.
    const int j = lane & 31;            // score operand row
    const int hsel = lane >> 5;         // which 8 of the MFMA's 16 k values
    // latent chunk (2ks + hsel) of row j sits at ((2ks + hsel) ^ swz(j)):
    // offset = sc_base ^ ((ks % 8) << 5), plus 256 bytes per 8 ks
    const int sc_base = j * 1024 + ((hsel ^ lat_swz(j)) << 4);
    // rotary chunk (2ks + hsel) of block row j%8 sits at ((2ks + hsel) ^ (j%8))
    const int pe_base = kLatBytes + (j >> 3) * kPeBlock + (j & 7) * 128 + ((hsel ^ (j & 7)) << 4);
    // transposing reads: 16-lane block blk reads rows 16kc + 8t + 4g + e4
    // (g = blk/2, e4 = (lane%16)/4) and columns 32cb + 16(blk%2) + 4(lane%4):
    // offset = tr_base[kc][t] ^ ((cb % 4) << 6), plus 256 bytes per 4 cb
    const int blk = lane >> 4, g = blk >> 1, e4 = (lane & 15) >> 2, q4 = lane & 3;
    const int lo = 2 * (blk & 1) + (q4 >> 1);
    int tr_base[2][2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int row = 16 * kc + 8 * t + 4 * g + e4;   // lat_swz(row) = 4*e4 + 2t + g
            tr_base[kc][t] = row * 1024 + (e4 << 6) + ((lo ^ (2 * t + g)) << 4) + (q4 & 1) * 8;
        }

    const lds_u8* tiles = (const lds_u8*)c.tiles;
    const unsigned tiles_addr = (unsigned)(size_t)c.tiles;
    const int jp = lane >> 3;                          // rotary row of this lane's gather
    const unsigned pe_lane = (unsigned)(((lane & 7) ^ jp) << 4);

    // Gathers.  Wave w fetches rows 8w .. 8w+7 of a tile: their latent parts
    // (eight 1 KiB loads) and their rotary parts (one load, lane l takes
    // 16 bytes of row 8w + l/8, whose index it reads itself).  A tile index
    // >= ntiles issues the same nine loads with out-of-range offsets (they
    // touch no memory), so every gather adds exactly nine to vmcnt.
    auto gather_index = [&](int t) -> int {
        return c.sidx[min(t, ntiles - 1) * kRows + 8 * c.wave + jp];
    };
    // Latent rows 8*wave + 4*g .. +3 of tile t, with one M0 value for the
    // four.  Their indices are adjacent in the LDS list: one broadcast read
    // gives all four to every lane (rows_index), and each row's offset is
    // plain vector arithmetic (row_offset), which the tile loop spreads over
    // several k-steps of the score chain.
    // The read's address goes through an opaque per-lane zero: the indices
    // are the same in every lane, and the compiler would otherwise move them
    // to scalar registers and test them there, a chain of lane-to-scalar
    // moves, scalar compares and vector selects that stalls the MFMA chain;
    // in vector registers each offset is three independent instructions.
    auto rows_index = [&](int t, int g) -> u32x4 {
        int lz = 0;
        asm volatile("" : "+v"(lz));
        return *(const __attribute__((address_space(3))) u32x4*)(
            (const __attribute__((address_space(3))) int*)c.sidx + min(t, ntiles - 1) * kRows + 8 * c.wave + 4 * g + lz);
    };
    auto row_offset = [&](int t, const u32x4& pv, int g, int u) -> unsigned {
        // one vector compare against a scalar limit (0 past the last tile);
        // the compiler would otherwise test the tile in a scalar mask and
        // combine the two, moving the condition between the units
        unsigned lim_t = t < ntiles ? lim : 0u;
        asm volatile("" : "+s"(lim_t));
        return x4_off(pv[u] < lim_t, (pv[u] << 10) + ((unsigned)(lane ^ lat_swz(8 * c.wave + 4 * g + u)) << 4), u);
    };
    auto issue_rows4 = [&](int t, int g, const unsigned (&v)[4]) {
        load_lds16_x4(c.kv_desc, tiles_addr + (t & (kBufs - 1)) * kBufBytes + (8 * c.wave + 4 * g) * 1024,
                      v[0], v[1], v[2], v[3]);
    };
    auto gather_rows4 = [&](int t, int g) {
        const u32x4 pv = rows_index(t, g);
        unsigned v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = row_offset(t, pv, g, u);
        issue_rows4(t, g, v);
    };
    auto gather_pe = [&](int t, int pidx) {
        const unsigned lim_t = t < ntiles ? lim : 0u;
        const unsigned off = (unsigned)pidx < lim_t ? (unsigned)pidx * 128u + pe_lane : kOutOfRange;
        load_lds16(c.pe_desc, tiles_addr + (t & (kBufs - 1)) * kBufBytes + kLatBytes + c.wave * kPeBlock,
                   off);
    };
    auto gather_tile = [&](int t) {
        gather_rows4(t, 0);
        gather_rows4(t, 1);
        gather_pe(t, gather_index(t));
    };

    // Score operand (A) for k-step ks of the tile in buffer offset bo.
    auto sc_read = [&](int bo, int ks) -> bf16x8 {
        if (ks < 32)
            return *(const __attribute__((address_space(3))) bf16x8*)(
                tiles + (((sc_base + bo) ^ ((ks & 7) << 5)) + (ks >> 3) * 256));
        return *(const __attribute__((address_space(3))) bf16x8*)(tiles + ((pe_base + bo) ^ ((ks - 32) << 5)));
    };
    // Standalone score chain (first tile).
    // Standalone score chain (first tile); side(ks) runs after each MFMA.
    auto scores = [&](int t, f32x16& out, auto&& side) {
        const int bo = (t & (kBufs - 1)) * kBufBytes;
        f32x16 sacc;
        bf16x8 pre[kScDepth];
#pragma unroll
        for (int d = 0; d < kScDepth; ++d) pre[d] = sc_read(bo, d);
#pragma unroll
        for (int ks = 0; ks < 36; ++ks) {
            const bf16x8 av = pre[ks % kScDepth];
            if (ks + kScDepth < 36) pre[ks % kScDepth] = sc_read(bo, ks + kScDepth);
            if (ks == 0) mfma32_v_first(sacc, av, qf[0]);
            else if (ks < 35) mfma32_v(sacc, av, qf[ks]);
            else mfma32_v_last(out, sacc, av, qf[ks]);
            side(ks);
        }
    };

    // Softmax bookkeeping of tile t, before its exponentials: mask the slots
    // that are not selected (only in partial tiles) and take the reference
    // from the first tile with a selected slot.  Returns the score multiplier
    // to use (1 once masking has applied the scale).
    bool have_ref = preset;
    // Read once: inside the loop the compiler would reload it from the
    // kernel arguments every tile (the assembly blocks clobber memory), and a
    // scalar load is waited for together with every LDS read in flight.
    const float scale_log2 = c.a->scale_log2;
    // `pv` is this lane's index list entry of tile t (row j), read ahead.
    auto prepare = [&](int t, f32x16& s, int pv) -> float {
        const unsigned vmask = (unsigned)__builtin_amdgcn_ballot_w64((unsigned)pv < lim);
        float sc = scale_log2;
        if (vmask != 0xFFFFFFFFu) {
            // this lane's rows are 8*(i/4) + 4*hsel + i%4
            const unsigned vml = vmask >> (4 * hsel);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const bool ok = (vml >> (8 * (i >> 2) + (i & 3))) & 1u;
                s[i] = ok ? s[i] * sc : -INFINITY;
            }
            sc = 1.f;
        }
        if (!have_ref && vmask != 0u) {
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i] * sc);
            m_ref = pair_max(mx);                    // a head spans lanes l and l ^ 32
            have_ref = true;
        }
        return sc;
    };
    // Probability of element i: 2^(s*sc - m_ref), into the bf16 B operand.
    auto prob = [&](const f32x16& s, int i, float sc, float neg_m, bf16x8 (&pb)[2], float& psum) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[i], sc, neg_m));
        psum += p;
        pb[i >> 3][i & 7] = (__bf16)p;
    };
    auto close_sum = [&](float psum) {
        l_run += psum;
        beaten = beaten || !(psum <= kRerunSum);
    };

    // Mix of the wave's own heads over all 512 latent columns, one tile:
    // O~^T[c][h] += V^T[c][j] P^T[j][h], c = 32*cb + (0..31), acc[cb].  Lane
    // (head h, half g) holds in pb[kc] the probabilities of rows
    // 16kc + 8t + 4g + e (slot 4t + e), which is exactly its share of the
    // B operand of k-step kc.  V^T is read kMixDepth MFMAs ahead; before(i)
    // runs ahead of MFMAs 4i .. 4i+3 and after(i) behind them.  Every MFMA
    // with its reads and hooks forms its own scheduling region, so that the
    // compiler cannot bunch the independent work between two MFMAs.
    auto mix = [&](int t, const bf16x8 (&pbm)[2], auto&& before, auto&& after) {
        const int bo = (t & (kBufs - 1)) * kBufBytes;
        auto v_read = [&](int m) -> bf16x8 {      // m = 16*kc + cb
            const int kc = m >> 4, cb = m & 15;
            const int x = (cb & 3) << 6, y = (cb >> 2) * 256;
            return cat(lds_read_tr(tiles + (((tr_base[kc][0] + bo) ^ x) + y)),
                       lds_read_tr(tiles + (((tr_base[kc][1] + bo) ^ x) + y)));
        };
        bf16x8 va[kMixDepth];
        if constexpr (!kMaxOnly) {
#pragma unroll
            for (int d = 0; d < kMixDepth; ++d) va[d] = v_read(d);
        }
#pragma unroll
        for (int m = 0; m < 32; ++m) {
            if ((m & 3) == 0) before(m >> 2);
            if constexpr (!kMaxOnly) {
                const bf16x8 av = va[m % kMixDepth];
                if (m + kMixDepth < 32) va[m % kMixDepth] = v_read(m + kMixDepth);
                acc[m & 15] = mfma32(av, pbm[m >> 4], acc[m & 15]);
            }
            if ((m & 3) == 3) after(m >> 2);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Score operands of the next chain, read ahead (kept across iterations).
    bf16x8 pre[kScDepth];
    // Gather offsets of the next tile to fetch, computed during a mix (one
    // per mix step, where independent MFMAs leave issue slots) and used by
    // the next score chain.
    unsigned goff[2][4];
    u32x4 pv[2];
    auto read_rows = [&](int tg) {
        pv[0] = rows_index(tg, 0);
        pv[1] = rows_index(tg, 1);
    };
    auto offsets_step = [&](int tg, int idx) {
        const int gg = idx >> 2, u = idx & 3;
        goff[gg][u] = row_offset(tg, pv[gg], gg, u);
        asm volatile("" : "+v"(goff[gg][u]));
    };
    auto preload = [&](int t) {
        const int bo = (t & (kBufs - 1)) * kBufBytes;
#pragma unroll
        for (int d = 0; d < kScDepth; ++d) pre[d] = sc_read(bo, d);
    };
    // Hand-over to the next iteration, placed before the last MFMAs of a mix
    // so that they cover the latency of the next chain's first reads: own
    // gathers of tile tn landed (the tile after it may stay in flight), then
    // a barrier after which tile tn is complete and every wave is done
    // reading the mixed tile.
    // This lane's index entry of the tile whose softmax comes next (read
    // ahead of the operand reads, so that waiting for it does not wait for
    // them).
    int sel = c.sidx[j];
    auto hand_over = [&](int tn) {
        MLA_WAIT_VMCNT(9);
        barrier_lds();
        sel = c.sidx[(tn - 1) * kRows + j];
        preload(tn);
        asm volatile("" ::: "memory");   // issue the reads here, not at their first use
    };

    // Iteration t with a next tile (tile t+1 complete and its first operands
    // read ahead): scores of t+1 into snext, softmax of t from scur, gather
    // of t+3, then the mix of t, with the hand-over to iteration t+1.
    auto body = [&](int t, f32x16& scur, f32x16& snext) {
        const float sc = prepare(t, scur, sel);
        const float neg_m = have_ref ? -m_ref : 0.f;
        float mx = -INFINITY;            // max-only passes
        const int bo = ((t + 1) & (kBufs - 1)) * kBufBytes;
        const int pidx = gather_index(t + 3);
        bf16x8 pb[2];
        float psum = 0.f;
        f32x16 sacc;
#pragma unroll
        for (int ks = 0; ks < 36; ++ks) {
            const bf16x8 av = pre[ks % kScDepth];
            if (ks + kScDepth < 36) pre[ks % kScDepth] = sc_read(bo, ks + kScDepth);
            if (ks == 0) mfma32_v_first(sacc, av, qf[0]);
            else if (ks < 35) mfma32_v(sacc, av, qf[ks]);
            else mfma32_v_last(snext, sacc, av, qf[ks]);
            // one exponential every other k-step, so that each fits in the
            // shadow of the MFMA in flight; each k-step is a scheduling
            // region of its own, or the compiler bunches the exponentials
            if constexpr (kMaxOnly) {
                if (ks < 16) mx = fmaxf(mx, scur[ks] * sc);
            } else {
                if (ks < 32 && !(ks & 1)) prob(scur, ks >> 1, sc, neg_m, pb, psum);
            }
            if (ks == 18) issue_rows4(t + 3, 0, goff[0]);
            if (ks == 26) issue_rows4(t + 3, 1, goff[1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (kMaxOnly) l_run = fmaxf(l_run, mx);
        else close_sum(psum);
        mix(t, pb, [&](int idx) {
                   if (idx == 0) read_rows(t + 4);
                   if (idx == 7) hand_over(t + 2);
               },
               [&](int idx) {
                   if (idx == 3) gather_pe(t + 3, pidx);
                   offsets_step(t + 4, idx);
               });
    };
    // Last tile: softmax and mix only.
    auto last = [&](int t, f32x16& scur) {
        const float sc = prepare(t, scur, sel);
        const float neg_m = have_ref ? -m_ref : 0.f;
        bf16x8 pb[2];
        float psum = 0.f;
        if constexpr (kMaxOnly) {
#pragma unroll
            for (int i = 0; i < 16; ++i) l_run = fmaxf(l_run, scur[i] * sc);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) prob(scur, i, sc, neg_m, pb, psum);
            close_sum(psum);
        }
        mix(t, pb, [](int) {}, [](int) {});
    };

    // The first score chain needs the query fragments and tile 0 only.  Tile
    // 1 is gathered right behind tile 0 (groups under different M0 values go
    // out a short sleep apart: back to back, each would wait for the one
    // before it), so that it is in flight while the chain runs; one wait then
    // leaves only tile 1's nine loads outstanding: the query fragments, which
    // were loaded first, and tile 0 have landed.  The compiler does not see
    // the gathers (inline assembly) and takes the last query loads for
    // pending, so its own waits in the chain's last k-steps also wait for tile
    // 1, which the loop needs next anyway.  Tile 2 goes out after the chain
    // (the compiler has no load of its own pending then), ahead of the
    // hand-over, whose wait then leaves tile 2 in flight as in the loop.
    gather_tile(0);
    __builtin_amdgcn_s_sleep(2);
    gather_rows4(1, 0);
    __builtin_amdgcn_s_sleep(2);
    gather_rows4(1, 1);
    __builtin_amdgcn_s_sleep(2);
    gather_pe(1, gather_index(1));
    MLA_WAIT_VMCNT(9);
    barrier_only();
    f32x16 sA, sB;
    scores(0, sA, [&](int) {});
    gather_rows4(2, 0);
    __builtin_amdgcn_s_sleep(2);
    gather_rows4(2, 1);
    __builtin_amdgcn_s_sleep(2);
    gather_pe(2, gather_index(2));
    if (ntiles > 1) hand_over(1);
    read_rows(3);
#pragma unroll
    for (int idx = 0; idx < 8; ++idx) offsets_step(3, idx);
    int t = 0;
    for (; t + 1 < ntiles; ++t) {
        body(t, sA, sB);
        sA = sB;
    }
    last(t, sA);
    MLA_WAIT_VMCNT(0);                   // no gather may land after the workgroup ends
    if constexpr (kMaxOnly) m_ref = pair_max(l_run);   // a head spans lanes l and l ^ 32
}

// Write this split's mix in bf16, not normalised (+ reference and sum; the
// merge divides by the total sum, so the normalisation costs no work here,
// where it would be 256 multiplies per lane at the end of the kernel).  Each
// wave holds all 512 columns of its own 32 heads (a head's columns split
// between lanes l and l ^ 32).  Rows are staged in LDS (the tile buffers are
// free once every wave is done with them) and every head row is written with
// one 1 KiB store instruction: stores straight from the accumulator layout
// would write sixteen scattered 16-byte pieces per instruction, and the
// memory system's cost goes with the number of pieces.  A wave stages and
// stores only its own heads' rows, and its LDS accesses run in order, so no
// barrier separates the two.
constexpr int kOutRow = 1040;   // staged output row: 512 bf16 + 16 bytes (spreads banks)

__device__ __forceinline__ void attn_finish(const SplitCtx& c, const f32x16 (&acc)[16], float m_ref,
                                            float l_run) {
    const AttnArgs& a = *c.a;
    const int lane = lane_id();
    const float l_tot = pair_sum(l_run);                 // a head spans lanes l and l ^ 32
    const int h_own = 32 * c.wave + (lane & 31);
    // (the caller has passed a barrier after every wave is done with the tiles)

    // acc[cb] element i: head h_own, column 32*cb + 8*(i/4) + 4*(lane/32) + i%4.
    // A quarter of the columns at a time: the stores of one quarter drain
    // while the next is staged.
    unsigned char* mine = c.tiles + h_own * kOutRow + 8 * (lane >> 5);
    __bf16* dst0 = reinterpret_cast<__bf16*>(a.o) + (((size_t)c.split * a.R + c.r) * kHeads + 32 * c.wave) * kLatent;
    const unsigned char* stage = c.tiles + 32 * c.wave * kOutRow;
#pragma unroll
    for (int qc = 0; qc < 4; ++qc) {
#pragma unroll
        for (int cb = 4 * qc; cb < 4 * qc + 4; ++cb)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const f32x16& v = acc[cb];
                *reinterpret_cast<bf16x4*>(mine + 64 * cb + 16 * gq) =
                    to_bf16x4(v[4 * gq], v[4 * gq + 1], v[4 * gq + 2], v[4 * gq + 3]);
            }
        // 32 head rows x 256 bytes: lane l takes row 4s + l/16, bytes 16(l%16) .. +15 of the quarter
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int row = 4 * s + (lane >> 4);
            const u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * kOutRow + 256 * qc + 16 * (lane & 15));
            *reinterpret_cast<u32x4*>(dst0 + (size_t)row * kLatent + 128 * qc + 8 * (lane & 15)) = v;
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (lane < 32) {
        const size_t orow = ((size_t)c.split * a.R + c.r) * kHeads + h_own;
        a.m_part[orow] = m_ref;
        a.l_part[orow] = l_tot;
    }
}

// The arguments a workgroup needs before its first loads.  The attention and
// merge kernels take them as leading scalar parameters, which the build has
// the compiler preload into scalar registers (-amdgpu-kernarg-preload-count):
// a workgroup then issues its first loads without first waiting for a
// kernel-argument load.  The full argument block follows them for everything
// needed later.
struct AttnEarly {
    const void* kv;
    const void* pe;
    const int32_t* idx;
    const void* q;
    int R, T, k, n_split, slots_per_split, causal_base;
    long long cache_rows_per_query;
};

// Workgroup slot -> (query row, split).  Consecutive slots land on the 8 XCDs
// in turn; the splits of one query row share an XCD, so its absorbed query is
// read from HBM once.  Latest query rows (most work) go first.  Returns false
// for a slot past the last row.
template <bool kRowMajor>
__device__ __forceinline__ bool attn_setup(SplitCtx& c, const AttnArgs& args, const AttnEarly& a, int id,
                                           unsigned char* tiles, int* sidx) {
    const int split = (id >> 3) % a.n_split;
    const int rr = ((id >> 3) / a.n_split) * 8 + (id & 7);
    if (rr >= a.R) return false;
    c.a = &args;
    c.tiles = tiles;
    c.sidx = sidx;
    c.r = (a.R - 1) - rr;
    c.split = split;
    c.wave = wave_id();
    c.lane = threadIdx.x & 63;
    const int slot_begin = split * a.slots_per_split;
    const int nslots = min(a.k, slot_begin + a.slots_per_split) - slot_begin;   // >= 1
    c.ntiles = (nslots + kRows - 1) / kRows;
    c.limit = a.causal_base < 0 ? 0x7fffffff : a.causal_base + c.r;
    c.T = a.T;
    c.kv_desc = make_desc_x4(reinterpret_cast<const __bf16*>(a.kv) + (size_t)c.r * a.cache_rows_per_query * kLatent,
                             (unsigned)c.T * (kLatent * 2));
    c.pe_desc = make_desc(reinterpret_cast<const __bf16*>(a.pe) + (size_t)c.r * a.cache_rows_per_query * kRope,
                          (unsigned)c.T * (kRope * 2));
    c.qrow = reinterpret_cast<const __bf16*>(a.q) + q_off(c.r, 32 * c.wave + (c.lane & 31), 8 * (c.lane >> 5), kRowMajor);
    c.idx_src = a.idx + (size_t)c.r * a.k + slot_begin;
    c.nslots = nslots;
    return true;
}

// LDS of the attention pass: tile buffers, the split's index list and each
// wave's last selected slot.
constexpr int kAttnTilesLds = kBufs * kBufBytes;
constexpr int kAttnLds = kAttnTilesLds + kMaxSlotsPerSplit * 4 + 8 * 4;   // + per wave: last selected slot, rerun flag
static_assert(kAttnLds <= 160 * 1024, "attention LDS exceeds a compute unit's 160 KiB");

// kRowMajor: the absorbed queries are row-major (R >= kQRowMajorMinRows), else the operand image.
template <bool kRowMajor>
__global__ __launch_bounds__(256, 1) void attn_bf16(const void* kv, const void* pe, const int32_t* idx,
                                                    const void* q, int R, int T, int k, int n_split,
                                                    int slots_per_split, int causal_base,
                                                    long long cache_rows_per_query, AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kAttnLds];
    SplitCtx c;
    const AttnEarly early{kv, pe, idx, q, R, T, k, n_split, slots_per_split, causal_base, cache_rows_per_query};
    if (!attn_setup<kRowMajor>(c, a, early, blockIdx.x, lds, reinterpret_cast<int*>(lds + kAttnTilesLds)))
        return;
    f32x16 acc[16];
    float m_ref = -INFINITY, l_run = 0.f;
    bool beaten;
    attn_pass<false, kRowMajor>(c, m_ref, acc, l_run, beaten, false);
    // A split in which a later score beat its head's reference by about 60
    // (log2 units) runs again, by every wave: a pass that finds each head's
    // largest score, then the full pass with it as the reference (never the
    // case for realistic attention; the benchmark times a forced case).
    int* any_beaten = reinterpret_cast<int*>(lds + kAttnTilesLds) + kMaxSlotsPerSplit + 4;
    const bool wave_beaten = __builtin_amdgcn_ballot_w64(beaten) != 0;   // every lane takes part
    if (lane_id() == 0) any_beaten[c.wave] = wave_beaten;
    barrier_lds();                       // also: every wave is done with the tiles
    if (any_beaten[0] | any_beaten[1] | any_beaten[2] | any_beaten[3]) {
        attn_pass<true, kRowMajor>(c, m_ref, acc, l_run, beaten, true);
        barrier_lds();                   // every wave is done with the tiles
        attn_pass<false, kRowMajor>(c, m_ref, acc, l_run, beaten, true);
        if (c.wave == 0 && lane_id() == 0) atomicAdd(a.stats, 1);
        barrier_lds();                   // every wave is done with the tiles
    }
    attn_finish(c, acc, m_ref, l_run);
}

// --------------------------------------------------------------------------
// Step 4 merge + step 5: out[r, h, :] = O~[r, h, :] . W_UV[h]^T
//
// Per head a [R x 512] . [512 x 128] product, computed transposed:
// out^T = W_UV[h] . O~^T, with W_UV rows (d) as the A operand in registers.
// Workgroup = (head, group of 32-row query blocks); wave w owns output values
// d = 32w .. 32w+31.  Each wave merges eight rows of the block: all of its partial loads are
// issued at once (loads of every split of a row land while the weights are
// computed), merged in float32 with w_s = 2^(m_s - M) / sum_s' l_s' 2^(m_s' - M)
// (M: the largest reference among splits with a selected slot; a split with
// l_s = 0 weighs 0) and stored to LDS as bf16, swizzled as the attention
// tiles are; after a barrier every wave multiplies the 32 merged rows.
// --------------------------------------------------------------------------
constexpr int kUvRows = 32;
constexpr int kUvChunk = 4;                    // splits whose loads are in flight together
constexpr int kUvLds = kUvRows * 1024;

// Wave w's slice of W_UV[h] (rows d = 32w .. 32w+31) as MFMA A fragments:
// k-step ks, lane half g takes columns 16ks + 8g .. +7.  The slice is read as
// whole 128-byte lines (load (i, m): rows 8i + lane/8, bytes 128m + 16(lane%8)
// .. +15) into the wave's own LDS rows (1040-byte stride: the 16-byte fragment
// reads of 32 rows fall in distinct banks), then read back as fragments.
// Reading the fragments straight from memory takes 32 bytes from each of 32
// rows per load instruction, which the memory pipeline serves at about half
// the rate of whole lines.
constexpr int kUvWRow = 1040;
constexpr int kUvWLds = 4 * 32 * kUvWRow;
__device__ __forceinline__ void uv_load_w(const __bf16* __restrict__ w_uv, int h, bf16x8 (&wa)[32],
                                          unsigned char* stage) {
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    unsigned char* mine = stage + wave * 32 * kUvWRow;
    const unsigned char* src = reinterpret_cast<const unsigned char*>(w_uv + ((size_t)h * kValue + 32 * wave) * kLatent);
    const int r8 = lane >> 3, b16 = 16 * (lane & 7);
#pragma unroll
    for (int part = 0; part < 2; ++part) {
        u32x4 v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int i = (16 * part + q) >> 3, m = q & 7;
            v[q] = *reinterpret_cast<const u32x4*>(src + (size_t)(8 * i + r8) * (kLatent * 2) + 128 * m + b16);
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int i = (16 * part + q) >> 3, m = q & 7;
            *reinterpret_cast<u32x4*>(mine + (8 * i + r8) * kUvWRow + 128 * m + b16) = v[q];
        }
    }
    const unsigned char* frag = mine + (lane & 31) * kUvWRow + 16 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) wa[ks] = *reinterpret_cast<const bf16x8*>(frag + 32 * ks);
}

// Merge + W_UV of head h for query rows 32*rb .. 32*rb + 31.  Every thread of
// the workgroup calls it; `lds` holds kUvLds bytes (1 KiB aligned).
// kManySplits: more than eight splits (each lane then combines several pairs).
template <bool kManySplits>
__device__ __forceinline__ void uv_block(const __bf16* __restrict__ o_ws, const float* __restrict__ m_part,
                                         const float* __restrict__ l_part, __bf16* __restrict__ out, int R,
                                         int n_split, int h, int rb, const bf16x8 (&wa)[32],
                                         unsigned char* lds) {
    const int wave = wave_id();
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    const size_t split_stride = (size_t)R * kHeads;           // partial rows between splits
    const int r0 = rb * kUvRows + 8 * wave;                    // this wave's first row
    const int nr = max(0, min(8, R - r0));                     // its rows inside R

    // Merge weights, computed while the first partial loads are in flight.
    // Lane l works on row jj = l / 8 of the wave's eight rows and on the
    // splits s with s % 8 == l % 8; the eight lanes of a row then combine
    // their (reference, sum) pairs into the row's largest reference M and
    // the inverse of its total weight sum_s l_s 2^(m_s - M).  Each lane's
    // first pair (split l % 8, kept for the first chunk's weights below) is
    // loaded ahead of the partials, from a row and split clamped into range.
    const int wj = lane >> 3, wu = lane & 7;
    const bool wrow = wj < nr;
    const size_t wrow_off = (size_t)(r0 + (wrow ? wj : 0)) * kHeads + h;
    const size_t o_first = (size_t)min(wu, n_split - 1) * split_stride + (size_t)min(r0 + wj, R - 1) * kHeads + h;
    const float l_ld = l_part[o_first], m_ld = m_part[o_first];

    // This wave's partial rows of splits s0 .. s0+kUvChunk-1, 16 bytes per
    // lane and row: columns 8l .. 8l+7.  Every load is issued, from a row the
    // attention kernel wrote (split and row clamped into range), so that the
    // count of loads in flight does not depend on the sizes; past the last
    // split or past R the value carries merge weight 0.
    bf16x8 v[kUvChunk][8];
    auto issue = [&](int s0) {
#pragma unroll
        for (int u = 0; u < kUvChunk; ++u)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const size_t row = (size_t)min(s0 + u, n_split - 1) * split_stride +
                                   (size_t)min(r0 + jj, R - 1) * kHeads + h;
                v[u][jj] = *reinterpret_cast<const bf16x8*>(o_ws + row * kLatent + 8 * lane);
            }
    };
    issue(0);
    __builtin_amdgcn_sched_barrier(0);   // the partial loads go out before the weights are computed

    const bool first_ok = wrow && wu < n_split;
    const float l_first = first_ok ? l_ld : 0.f, m_first = first_ok ? m_ld : -INFINITY;
    float mrow = -INFINITY, lrow = 0.f;
    if (l_first > 0.f) {
        mrow = m_first;
        lrow = l_first;
    }
    // (with at most eight splits there is nothing more, and the compiler's
    // count of loads in flight stays exact: the weights below then need only
    // the pairs, not the partials)
    if constexpr (kManySplits) {
        for (int sp = wu + 8; sp < n_split; sp += 8) {
            const float l = wrow ? l_part[sp * split_stride + wrow_off] : 0.f;
            const float m = wrow ? m_part[sp * split_stride + wrow_off] : -INFINITY;
            if (l > 0.f) {
                const float mn = fmaxf(mrow, m);
                lrow = lrow * exp2f(mrow - mn) + l * exp2f(m - mn);
                mrow = mn;
            }
        }
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
        const float m2 = __shfl_xor(mrow, o), l2 = __shfl_xor(lrow, o);
        const float mn = fmaxf(mrow, m2);
        lrow = (lrow > 0.f ? lrow * exp2f(mrow - mn) : 0.f) + (l2 > 0.f ? l2 * exp2f(m2 - mn) : 0.f);
        mrow = mn;
    }
    const float inv_row = lrow > 0.f ? 1.f / lrow : 0.f;

    // Merged rows: lane l holds columns 8l .. 8l+7 of each of its rows.
    float x[8][8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[jj][e] = 0.f;
    // One chunk of kUvChunk splits: the weight of split s0 + (l % 8) for row
    // l / 8 from its pair (lanes with l % 8 >= kUvChunk idle), broadcast to
    // the rows' lanes.  The first chunk is straight-line code (its pairs are
    // the ones read above), so that its multiply-adds wait for each partial
    // load as it lands; later chunks (more than four splits) read their pairs,
    // both values at once.
    auto merge_chunk = [&](int s0, float l, float m) {
        float w = 0.f;
        if (wrow && wu < kUvChunk && s0 + wu < n_split) w = l > 0.f ? exp2f(m - mrow) * inv_row : 0.f;
#pragma unroll
        for (int u = 0; u < kUvChunk; ++u)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const float wv = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), 8 * jj + u));
#pragma unroll
                for (int e = 0; e < 8; ++e) x[jj][e] = fmaf(wv, (float)v[u][jj][e], x[jj][e]);
            }
    };
    merge_chunk(0, l_first, m_first);
    for (int s0 = kUvChunk; s0 < n_split; s0 += kUvChunk) {
        issue(s0);
        const size_t o = (size_t)min(s0 + wu, n_split - 1) * split_stride + wrow_off;
        merge_chunk(s0, l_part[o], m_part[o]);
    }
    // Stage the merged rows (bf16) for the B operand: 16-byte chunk l of row j
    // at chunk (l & ~15) | ((l & 15) ^ lat_swz(j)).
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        const int j = 8 * wave + jj;
        bf16x8 b;
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = (__bf16)x[jj][e];
        *reinterpret_cast<bf16x8*>(lds + j * 1024 + (((lane & ~15) | ((lane & 15) ^ lat_swz(j))) << 4)) = b;
    }
    barrier_lds();

    // out^T[d][r] = sum_c W[d][c] O~[r][c]; B operand column r = lane % 32
    const int j = lane & 31;
    const int b_base = j * 1024 + ((half ^ lat_swz(j)) << 4);
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) {
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(lds + ((b_base ^ ((ks & 7) << 5)) + (ks >> 3) * 256));
        acc = mfma32(wa[ks], bv, acc);
    }
    const int r = rb * kUvRows + j;
    if (r < R) {
        __bf16* dst = out + ((size_t)r * kHeads + h) * kValue + 32 * wave + 4 * half;
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *reinterpret_cast<bf16x4*>(dst + 8 * g) = to_bf16x4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
    }
}

template <bool kManySplits>
__global__ __launch_bounds__(256, 1) void uv_bf16(const __bf16* __restrict__ o, const float* __restrict__ m_part,
                                                  const float* __restrict__ l_part,
                                                  const __bf16* __restrict__ w_uv, int R, int n_split,
                                                  int r_groups, __bf16* __restrict__ out) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kUvWLds > kUvLds ? kUvWLds : kUvLds];
    const int h = blockIdx.x;
    bf16x8 wa[32];
    uv_load_w(w_uv, h, wa, lds);
    __syncthreads();                     // every wave has its fragments before the merge staging reuses LDS
    for (int rb = blockIdx.y; rb * kUvRows < R; rb += r_groups) {
        if (rb != (int)blockIdx.y) barrier_only();       // the staging is reused by this block
        uv_block<kManySplits>(o, m_part, l_part, out, R, n_split, h, rb, wa, lds);
    }
}

// The same merge + W_UV when every row has one split (the prefill chunk's lists
// fit one): the merged row is the split's mix divided by its weight sum.
// Each wave's partial rows of the workgroup's next block are loaded while the
// current block is multiplied (two register sets, the loop taking blocks in
// pairs), so that a workgroup's blocks overlap instead of each waiting for its
// loads.  Past R, rows are loaded from row R - 1 and dropped.
__global__ __launch_bounds__(256, 1) void uv1_bf16(const __bf16* __restrict__ o, const float* __restrict__ l_part,
                                                   const __bf16* __restrict__ w_uv, int R, int r_groups,
                                                   __bf16* __restrict__ out) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kUvWLds > kUvLds ? kUvWLds : kUvLds];
    const int h = blockIdx.x;
    const int wave = wave_id();
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    bf16x8 wa[32];
    uv_load_w(w_uv, h, wa, lds);
    __syncthreads();                     // every wave has its fragments before the staging reuses LDS
    const int blocks = (R + kUvRows - 1) / kUvRows;
    // rows 32 rb + 8 wave + jj (jj < 8): lane l loads latent columns 8l .. 8l+7 of each, and the
    // weight sum of row 32 rb + 8 wave + l / 8
    auto load = [&](int rb, bf16x8 (&v)[8], float& l) {
        const int r0 = min(rb, blocks - 1) * kUvRows + 8 * wave;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            v[jj] = *reinterpret_cast<const bf16x8*>(o + ((size_t)min(r0 + jj, R - 1) * kHeads + h) * kLatent + 8 * lane);
        l = l_part[(size_t)min(r0 + (lane >> 3), R - 1) * kHeads + h];
    };
    auto process = [&](int rb, const bf16x8 (&v)[8], float l) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, inv), 8 * jj));
            const int j = 8 * wave + jj;
            bf16x8 b;
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = (__bf16)((float)v[jj][e] * w);
            *reinterpret_cast<bf16x8*>(lds + j * 1024 + (((lane & ~15) | ((lane & 15) ^ lat_swz(j))) << 4)) = b;
        }
        barrier_lds();
        const int j = lane & 31;
        const int b_base = j * 1024 + ((half ^ lat_swz(j)) << 4);
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) {
            const bf16x8 bv = *reinterpret_cast<const bf16x8*>(lds + ((b_base ^ ((ks & 7) << 5)) + (ks >> 3) * 256));
            acc = mfma32(wa[ks], bv, acc);
        }
        const int r = rb * kUvRows + j;
        if (r < R) {
            __bf16* dst = out + ((size_t)r * kHeads + h) * kValue + 32 * wave + 4 * half;
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<bf16x4*>(dst + 8 * g) = to_bf16x4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
        }
        barrier_only();                  // staging reused by the next block
    };
    bf16x8 va[8], vb[8];
    float la, lb;
    int rb = blockIdx.y;
    load(rb, va, la);
    for (; rb < blocks; rb += 2 * r_groups) {
        load(rb + r_groups, vb, lb);
        process(rb, va, la);
        if (rb + r_groups >= blocks) break;
        load(rb + 2 * r_groups, va, la);
        process(rb + r_groups, vb, lb);
    }
}

}  // namespace

hipError_t launch_absorb_bf16(const void* q_nope, const void* q_pe, const void* w_uk, void* q_out,
                              int R, int* stats, hipStream_t s) {
    // one workgroup per (head, quarter of c) and up to 64 query blocks: the
    // weight slice is read once per 64 blocks (at a 4096-query chunk, 8 blocks
    // per workgroup took the kernel 291 us, 64 take 245 us)
    const int blocks = (R + 31) / 32;
    const int r_groups = (blocks + 63) / 64;
    auto kernel = R >= kQRowMajorMinRows ? absorb_q_bf16<true> : absorb_q_bf16<false>;
    hipLaunchKernelGGL(kernel, dim3(kHeads * 4, r_groups), dim3(256), 0, s,
                       static_cast<const __bf16*>(q_nope), static_cast<const __bf16*>(q_pe),
                       static_cast<const __bf16*>(w_uk), static_cast<__bf16*>(q_out), R, r_groups, stats);
    return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
    const int row_groups = (a.R + 7) / 8;
    auto kernel = a.R >= kQRowMajorMinRows ? attn_bf16<true> : attn_bf16<false>;
    hipExtLaunchKernelGGL(kernel, dim3(row_groups * 8 * a.n_split), dim3(256), 0, s, start, stop, 0,
                          a.kv, a.pe, a.idx, a.q, a.R, a.T, a.k, a.n_split, a.slots_per_split, a.causal_base,
                          a.cache_rows_per_query, a);
    return hipGetLastError();
}

hipError_t launch_uv_bf16(const AttnArgs& a, const void* w_uv, void* out, hipStream_t s) {
    const int blocks = (a.R + 31) / 32;
    const int r_groups = blocks < 8 ? blocks : 8;
    if (a.n_split == 1) {
        hipLaunchKernelGGL(uv1_bf16, dim3(kHeads, r_groups), dim3(256), 0, s, static_cast<const __bf16*>(a.o),
                           a.l_part, static_cast<const __bf16*>(w_uv), a.R, r_groups, static_cast<__bf16*>(out));
        return hipGetLastError();
    }
    hipLaunchKernelGGL(a.n_split > 8 ? uv_bf16<true> : uv_bf16<false>, dim3(kHeads, r_groups), dim3(256), 0, s,
                       static_cast<const __bf16*>(a.o),
                       a.m_part, a.l_part, static_cast<const __bf16*>(w_uv), a.R, a.n_split, r_groups,
                       static_cast<__bf16*>(out));
    return hipGetLastError();
}

}  // namespace mla
