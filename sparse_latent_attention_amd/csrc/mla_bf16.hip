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

// Buffer resource over `bytes` bytes at `base`.  A raw buffer load whose
// offset is >= bytes returns zeros without touching memory; kOutOfRange is
// such an offset for every buffer these kernels build (<= 2 GiB).
constexpr unsigned kOutOfRange = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Layout of the absorbed queries in the workspace, chosen for the attention
// waves' score operands: element c (0..575: 512 latent, then 64 rotary) of
// head h of query row r sits at
//   ((r*4 + h/32)*36 + c/16)*512 + (h%32)*16 + c%16,
// so the 16-byte operand loads of one wave and k-step read one contiguous
// 1 KiB run, and the absorption writes 32-byte runs.
__device__ __forceinline__ size_t q_off(int r, int h, int c) {
    return (((size_t)r * 4 + (h >> 5)) * 36 + (c >> 4)) * 512 + (size_t)((h & 31) * 16) + (c & 15);
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
    auto load_q = [&](int rb, u32x4 (&p)[2]) {
        const int r = rb * 32 + (tid >> 3);
        const bool rv = r < R;
        const __bf16* qn = q_nope + ((size_t)(rv ? r : 0) * kHeads + h) * kNope + 16 * (tid & 7);
        p[0] = rv ? *reinterpret_cast<const u32x4*>(qn) : u32x4{};
        p[1] = rv ? *reinterpret_cast<const u32x4*>(qn + 8) : u32x4{};
    };
    auto stage_q = [&](const u32x4 (&p)[2], unsigned char* qb) {
        unsigned char* dst = qb + (tid >> 3) * kQnRow + 32 * (tid & 7);
        *reinterpret_cast<u32x4*>(dst) = p[0];
        *reinterpret_cast<u32x4*>(dst + 16) = p[1];
    };
    // B fragments of a staged block: q_nope[r][h][16ks + 8half .. +7], r = lane % 32
    auto frags_q = [&](const unsigned char* qb, bf16x8 (&b)[8]) {
        const unsigned char* src = qb + (lane & 31) * kQnRow + 16 * half;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) b[ks] = *reinterpret_cast<const bf16x8*>(src + 32 * ks);
    };
    const int blocks = (R + 31) / 32;
    bf16x8 b0[8], b1[8];
    u32x4 p0[2], p1[2];
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
    stage_q(p0, qbuf[0]);
    if (rb_first + r_groups < blocks) stage_q(p1, qbuf[1]);
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

    auto process = [&](int rb, const bf16x8 (&b)[8]) {
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
                *reinterpret_cast<u32x4*>(q_out + q_off(rr, h, cq * 128 + 8 * (e & 15))) =
                    *reinterpret_cast<const u32x4*>(obuf + (e >> 4) * kQcRow + 16 * (e & 15));
        }
        if (cq == 0) {
            // q_pe rows of this block: 32 rows x 8 chunks of 16 bytes = one per thread.
            const int rr = rb * 32 + (tid >> 3);
            const int ch = tid & 7;
            if (rr < R) {
                *reinterpret_cast<bf16x8*>(q_out + q_off(rr, h, kLatent + 8 * ch)) =
                    *reinterpret_cast<const bf16x8*>(q_pe + ((size_t)rr * kHeads + h) * kRope + 8 * ch);
            }
        }
        __syncthreads();                  // obuf reused by the next block
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
        process(rb, b0);
        if (more0) stage_q(p0, qbuf[0]);
        if (has1) {
            if (more1) load_q(rb + 3 * r_groups, p1);
            process(rb + r_groups, b1);
            if (more1) stage_q(p1, qbuf[1]);
        }
        if (more0) {
            __syncthreads();              // staged blocks visible
            frags_q(qbuf[0], b0);
            if (more1) frags_q(qbuf[1], b1);
        }
    }
}

__global__ __launch_bounds__(256) void absorb_q_bf16(const __bf16* __restrict__ q_nope,
                                                     const __bf16* __restrict__ q_pe,
                                                     const __bf16* __restrict__ w_uk,
                                                     __bf16* __restrict__ q_out, int R,
                                                     int r_groups) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kAbsorbLds];
    // Workgroups are dealt to the eight XCDs in turn (id % 8).  XCD x takes
    // heads 16x .. 16x+15 with all four column quarters, so a head's queries
    // come from memory once per launch (the other quarters hit that XCD's L2)
    // and the 32-byte output pieces of neighbouring heads, which share cache
    // lines, are merged in one L2 before they are written back.
    const int b = blockIdx.x, j = b >> 3;
    absorb_unit(q_nope, q_pe, w_uk, q_out, R, (16 * (b & 7) + (j >> 2)) * 4 + (j & 3), blockIdx.y,
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
//            accumulator is never rescaled (which keeps it in the accumulation
//            registers); if a head's probabilities in one tile sum past 2^32
//            (a later score beat m by about 32), which no realistic attention
//            does, the head is flagged and the merge recomputes it exactly;
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
    const __bf16* qrow;          // this lane's score operands: k-step ks at qrow + 512*ks
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

// A head whose per-tile probability sum exceeds this (relative to its
// reference) is recomputed exactly by the merge; below it, no probability or
// partial sum comes near the float/bf16 range.
constexpr float kBeatenSum = 4294967296.f;   // 2^32

// One pass over the split's tiles.  Software pipeline, per iteration t: the
// score MFMAs of tile t+1 run with the softmax of tile t and the gathers of
// tile t+3 interleaved between them (VALU and memory instructions issue while
// an MFMA executes), then the mix MFMAs of tile t, with the hand-over to the
// next iteration (own gathers of tile t+2 landed, then a barrier) before its
// last four MFMAs.
// The reference of each head is the (scaled) maximum of its first tile with
// a selected row; no rescaling happens afterwards.  `beaten` reports a tile
// whose probabilities exceeded kBeatenSum against that reference.
__device__ __forceinline__ void attn_pass(const SplitCtx& c, float& m_ref, f32x16 (&acc)[16],
                                          float& l_run, bool& beaten) {
    const int lane = c.lane;
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
    for (int ks = 0; ks < 36; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(c.qrow + 512 * ks);
    // The split's last selected slot: tiles past it hold no selected row (a
    // causal prefill query early in its chunk leaves most of its list empty)
    // and are not processed.
    int last_sel = -1;
#pragma unroll
    for (int u = 0; u < kIdxPerThread; ++u) {
        const int i = (int)threadIdx.x + 256 * u;
        if (i < c.nslots && (unsigned)iv[u] < lim) last_sel = i;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) last_sel = max(last_sel, __shfl_xor(last_sel, o));
    if (lane == 0) c.sidx[kMaxSlotsPerSplit + c.wave] = last_sel;
#pragma unroll
    for (int u = 0; u < kIdxPerThread; ++u) {
        const int i = (int)threadIdx.x + 256 * u;
        if (i < c.ntiles * kRows) c.sidx[i] = iv[u];
    }
    barrier_lds();
    const int* wave_last = c.sidx + kMaxSlotsPerSplit;
    const int ntiles = (max(max(wave_last[0], wave_last[1]), max(wave_last[2], wave_last[3])) + kRows) / kRows;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) acc[cb] = f32x16{};
    l_run = 0.f;
    if (ntiles == 0) {                   // nothing selected: an empty partial
        __builtin_amdgcn_s_waitcnt(0);   // no load may land after the workgroup ends
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
    bool have_ref = false;
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
            m_ref = fmaxf(mx, __shfl_xor(mx, 32));   // a head spans lanes l and l ^ 32
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
        beaten = beaten || !(psum <= kBeatenSum);
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
#pragma unroll
        for (int d = 0; d < kMixDepth; ++d) va[d] = v_read(d);
#pragma unroll
        for (int m = 0; m < 32; ++m) {
            const bf16x8 av = va[m % kMixDepth];
            if (m + kMixDepth < 32) va[m % kMixDepth] = v_read(m + kMixDepth);
            if ((m & 3) == 0) before(m >> 2);
            acc[m & 15] = mfma32(av, pbm[m >> 4], acc[m & 15]);
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
            if (ks < 32 && !(ks & 1)) prob(scur, ks >> 1, sc, neg_m, pb, psum);
            if (ks == 32) close_sum(psum);
            if (ks == 18) issue_rows4(t + 3, 0, goff[0]);
            if (ks == 26) issue_rows4(t + 3, 1, goff[1]);
            __builtin_amdgcn_sched_barrier(0);
        }
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
#pragma unroll
        for (int i = 0; i < 16; ++i) prob(scur, i, sc, neg_m, pb, psum);
        close_sum(psum);
        mix(t, pb, [](int) {}, [](int) {});
    };

    // The first score chain needs the query fragments and tile 0 only.  The
    // wait for them is a full one: the compiler does not see the gathers
    // (inline assembly), so after a partial wait it would still take the
    // later query loads for pending and wait again inside the first score
    // chain, on counts that include the gathers of tiles 1 and 2.  Those go
    // out during that chain, spread over its k-steps rather than back to
    // back, so that its MFMAs cover their issue.
    gather_tile(0);
    __builtin_amdgcn_s_waitcnt(0);
    barrier_only();
    f32x16 sA, sB;
    scores(0, sA, [&](int ks) {
        if (ks == 2) gather_rows4(1, 0);
        if (ks == 8) gather_rows4(1, 1);
        if (ks == 14) gather_pe(1, gather_index(1));
        if (ks == 20) gather_rows4(2, 0);
        if (ks == 26) gather_rows4(2, 1);
        if (ks == 32) gather_pe(2, gather_index(2));
    });
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
}

// Write this split's mix in bf16, not normalised (+ reference and sum; the
// merge divides by the total sum, so the normalisation costs no work here,
// where it would be 256 multiplies per lane at the end of the kernel).  Each
// wave holds all 512 columns of its own 32 heads (a head's columns split
// between lanes l and l ^ 32).  Rows are staged in LDS (the tile buffers are
// free once every wave is done with them) and every head row is written with
// one 1 KiB store instruction.
constexpr int kOutRow = 1040;   // staged output row: 512 bf16 + 16 bytes (spreads banks)

__device__ __forceinline__ void attn_finish(const SplitCtx& c, const f32x16 (&acc)[16], float m_ref,
                                            float l_run, bool beaten) {
    const AttnArgs& a = *c.a;
    const int lane = c.lane;
    const float l_tot = l_run + __shfl_xor(l_run, 32);   // a head spans lanes l and l ^ 32
    const int h_own = 32 * c.wave + (lane & 31);
    barrier_only();                                      // every wave is done with the tiles

    // acc[cb] element i: head h_own, column 32*cb + 8*(i/4) + 4*(lane/32) + i%4.
    unsigned char* mine = c.tiles + h_own * kOutRow + 8 * (lane >> 5);
#pragma unroll
    for (int cb = 0; cb < 16; ++cb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const f32x16& v = acc[cb];
            *reinterpret_cast<bf16x4*>(mine + 64 * cb + 16 * gq) =
                to_bf16x4(v[4 * gq], v[4 * gq + 1], v[4 * gq + 2], v[4 * gq + 3]);
        }
    barrier_lds();
    __bf16* dst0 = reinterpret_cast<__bf16*>(a.o) + (((size_t)c.split * a.R + c.r) * kHeads + 32 * c.wave) * kLatent;
    const unsigned char* stage = c.tiles + 32 * c.wave * kOutRow;
#pragma unroll 8
    for (int row = 0; row < 32; ++row) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * kOutRow + 16 * lane);
        *reinterpret_cast<u32x4*>(dst0 + (size_t)row * kLatent + 8 * lane) = v;
    }
    // A head whose probabilities outgrew its reference is marked with a
    // negative sum; the merge recomputes it exactly.
    beaten = beaten || __shfl_xor((int)beaten, 32);
    if (lane < 32) {
        const size_t orow = ((size_t)c.split * a.R + c.r) * kHeads + h_own;
        a.m_part[orow] = m_ref;
        a.l_part[orow] = beaten ? -1.f : l_tot;
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
    c.qrow = reinterpret_cast<const __bf16*>(a.q) + q_off(c.r, 32 * c.wave + (c.lane & 31), 8 * (c.lane >> 5));
    c.idx_src = a.idx + (size_t)c.r * a.k + slot_begin;
    c.nslots = nslots;
    return true;
}

// LDS of the attention pass: tile buffers, the split's index list and each
// wave's last selected slot.
constexpr int kAttnTilesLds = kBufs * kBufBytes;
constexpr int kAttnLds = kAttnTilesLds + kMaxSlotsPerSplit * 4 + 4 * 4;   // + each wave's last selected slot
static_assert(kHeads * kOutRow <= kAttnTilesLds, "output staging must fit in the tile buffers");
static_assert(kAttnLds <= 160 * 1024, "attention LDS exceeds a compute unit's 160 KiB");

__global__ __launch_bounds__(256, 1) void attn_bf16(const void* kv, const void* pe, const int32_t* idx,
                                                    const void* q, int R, int T, int k, int n_split,
                                                    int slots_per_split, int causal_base,
                                                    long long cache_rows_per_query, AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kAttnLds];
    SplitCtx c;
    const AttnEarly early{kv, pe, idx, q, R, T, k, n_split, slots_per_split, causal_base, cache_rows_per_query};
    if (!attn_setup(c, a, early, blockIdx.x, lds, reinterpret_cast<int*>(lds + kAttnTilesLds)))
        return;
    f32x16 acc[16];
    float m_ref = -INFINITY, l_run = 0.f;
    bool beaten = false;
    attn_pass(c, m_ref, acc, l_run, beaten);
    attn_finish(c, acc, m_ref, l_run, beaten);
}

// --------------------------------------------------------------------------
// Step 4 merge + step 5: out[r, h, :] = O~[r, h, :] . W_UV[h]^T
//
// Per head a [R x 512] . [512 x 128] product, computed transposed:
// out^T = W_UV[h] . O~^T, so W_UV rows (d) are the A operand, loaded straight
// from HBM with 16-byte reads (c is contiguous in the weight).  Workgroup =
// (head, group of 32-row query blocks); wave w owns 32 values d and keeps its
// W_UV slice (32 x 512) in registers.
// Each 32-row block of O~ is built in LDS: the split partials of up to four
// splits at a time are loaded straight into LDS (latent chunk c of row j at
// the same swizzled position as in the attention tiles), merged in float32
// with weights w_s = 2^(m_s - max) / sum_s' l_s' 2^(m_s' - max) (the partials
// are not normalised), and written back as bf16 into the first split's rows,
// which then feed the MFMA B operand.
// --------------------------------------------------------------------------
constexpr int kUvRows = 32;
constexpr int kUvGroup = 4;                    // splits staged in LDS at a time
constexpr int kUvStage = kUvGroup * kUvRows * 1024;

// LDS byte offset of bf16 column col of staged row j (16-byte chunk swizzle).
__device__ __forceinline__ int uv_pos(int j, int col) {
    const int c8 = col >> 3;
    return j * 1024 + (((c8 & ~15) | ((c8 & 15) ^ lat_swz(j))) << 4) + ((col & 7) << 1);
}

// Exact mix of one (query row, head) in float32, for a head whose first-tile
// reference was beaten during the attention pass: pass one finds the maximum
// score over the row's whole index list, pass two weighs and mixes the
// selected latent rows (one 256-slot chunk at a time).  The result,
// normalised, is written to out[0..511].  All 256 threads take part.
__device__ void exact_mix(const AttnArgs& a, int rr, int h, float* out, float* red, float* p_s,
                          int* pos_s) {
    const int tid = threadIdx.x;
    const __bf16* qb = reinterpret_cast<const __bf16*>(a.q);
    const __bf16* kv = reinterpret_cast<const __bf16*>(a.kv) + (size_t)rr * a.cache_rows_per_query * kLatent;
    const __bf16* pe = reinterpret_cast<const __bf16*>(a.pe) + (size_t)rr * a.cache_rows_per_query * kRope;
    const int32_t* idx = a.idx + (size_t)rr * a.k;
    const int limit = a.causal_base < 0 ? 0x7fffffff : a.causal_base + rr;
    auto score = [&](int t) {
        float d = 0.f;
        for (int c = 0; c < kLatent; ++c) d += (float)qb[q_off(rr, h, c)] * (float)kv[(size_t)t * kLatent + c];
        for (int c = 0; c < kRope; ++c)
            d += (float)qb[q_off(rr, h, kLatent + c)] * (float)pe[(size_t)t * kRope + c];
        return d * a.scale_log2;
    };
    auto block_max = [&](float v) {
        for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
        __syncthreads();
        if ((tid & 63) == 0) red[tid >> 6] = v;
        __syncthreads();
        return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    };
    float m = -INFINITY;
    for (int base = 0; base < a.k; base += 256) {
        const int slot = base + tid;
        const int t = slot < a.k ? idx[slot] : -1;
        if (t >= 0 && t < a.T && t <= limit) m = fmaxf(m, score(t));
    }
    m = block_max(m);
    float acc0 = 0.f, acc1 = 0.f, lp = 0.f;
    for (int base = 0; base < a.k; base += 256) {
        const int slot = base + tid;
        int t = slot < a.k ? idx[slot] : -1;
        if (!(t >= 0 && t < a.T && t <= limit)) t = -1;
        const float p = t >= 0 ? exp2f(score(t) - m) : 0.f;
        lp += p;
        __syncthreads();
        p_s[tid] = p;
        pos_s[tid] = t;
        __syncthreads();
        for (int jj = 0; jj < 256; ++jj) {
            const int tj = pos_s[jj];
            if (tj < 0) continue;
            acc0 += p_s[jj] * (float)kv[(size_t)tj * kLatent + tid];
            acc1 += p_s[jj] * (float)kv[(size_t)tj * kLatent + tid + 256];
        }
    }
    for (int o = 32; o > 0; o >>= 1) lp += __shfl_xor(lp, o);
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = lp;
    __syncthreads();
    const float L = red[0] + red[1] + red[2] + red[3];
    const float inv = L > 0.f ? 1.f / L : 0.f;
    out[tid] = acc0 * inv;
    out[tid + 256] = acc1 * inv;
    __syncthreads();
}

// LDS of one merge + W_UV block: staged partials, then small per-row arrays.
constexpr int kUvSmall = (2 * kUvRows + kUvGroup * kUvRows + kUvRows + kLatent + 4 + 256 + 256) * 4;
constexpr int kUvLds = kUvStage + kUvSmall;

// Wave w's slice of W_UV[h] (rows d = 32w .. 32w+31) as MFMA A fragments.
__device__ __forceinline__ void uv_load_w(const __bf16* __restrict__ w_uv, int h, bf16x8 (&wa)[32]) {
    const int lane = threadIdx.x & 63;
    const int d = 32 * wave_id() + (lane & 31);
    const __bf16* wrow = w_uv + ((size_t)h * kValue + d) * kLatent + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) wa[ks] = *reinterpret_cast<const bf16x8*>(wrow + 16 * ks);
}

// The merge kernel's counterpart of AttnEarly: what a workgroup needs before
// its first loads, passed as leading scalar parameters.
struct UvEarly {
    const __bf16* o;
    const float* m_part;
    const float* l_part;
    int R, n_split;
};

// Merge + W_UV of head h for query rows 32*rb .. 32*rb + 31; `lds` holds kUvLds
// bytes (1 KiB aligned).  Every thread of the workgroup calls it.
template <bool kLoadW>
__device__ __forceinline__ void uv_block(const AttnArgs& a, const UvEarly& e, __bf16* __restrict__ out, int h, int rb,
                                         bf16x8 (&wa)[32], unsigned char* lds,
                                         const __bf16* __restrict__ w_uv) {
    unsigned char* stage = lds;
    float* s_mmax = reinterpret_cast<float*>(lds + kUvStage);
    float* s_inv = s_mmax + kUvRows;
    float (*s_w)[kUvRows] = reinterpret_cast<float (*)[kUvRows]>(s_inv + kUvRows);
    int* marked = reinterpret_cast<int*>(s_inv + kUvRows + kUvGroup * kUvRows);
    float* xo = reinterpret_cast<float*>(marked + kUvRows);
    float* xred = xo + kLatent;
    float* xp = xred + 4;
    int* xpos = reinterpret_cast<int*>(xp + 256);
    const int R = e.R;
    const int n_split = e.n_split;
    const int tid = threadIdx.x;
    const int wave = wave_id();
    const int lane = tid & 63;
    const int half = lane >> 5;
    const unsigned stage_addr = (unsigned)(size_t)stage;
    const __bf16* o_ws = e.o;

    // Partial rows (split g0 + wave, query row rb*32 + j) -> staged row
    // (wave, j); rows past R or splits past n_split load zeros.
    auto stage_group = [&](int rb, int g0) {
        const int sp = g0 + wave;
        int ln = lane;
        asm volatile("" : "+v"(ln));
        // rows j of split sp sit kHeads * kLatent bf16 apart in the workspace
        const bool sp_ok = sp < n_split;
        const __bf16* src0 = o_ws + (((size_t)(sp_ok ? sp : 0) * R + rb * kUvRows) * kHeads + h) * kLatent;
        const unsigned row_bytes = kHeads * kLatent * 2;
        const u32x4 desc = make_desc_x4(src0, sp_ok ? (unsigned)min(R - rb * kUvRows, kUvRows) * row_bytes : 0u);
#pragma unroll 2
        for (int j0 = 0; j0 < kUvRows; j0 += 4) {
            unsigned v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + u;
                const bool ok = sp_ok && rb * kUvRows + j < R;
                v[u] = x4_off(ok, (unsigned)j * row_bytes + (unsigned)(((ln & ~15) | ((ln & 15) ^ lat_swz(j))) << 4), u);
            }
            load_lds16_x4(desc, stage_addr + (wave * kUvRows + j0) * 1024, v[0], v[1], v[2], v[3]);
        }
    };
    // Merge weight of a split with reference m and sum l for a row with
    // maximum mm and inverse weight sum inv: l 2^(m - mm) inv; a split with no
    // selected slot (l = 0) or an inexact one (l < 0) weighs 0.
    // Weight of a split's (unnormalised) partial: 2^(m - mm) / (sum over the
    // splits of l 2^(m - mm)), with inv that sum's inverse.
    auto weight = [&](float m, float l, float mm, float inv) {
        return l > 0.f ? exp2f(m - mm) * inv : 0.f;
    };


    // merge lanes: thread -> staged row mj, chunks mp[i] = 8i + (tid % 8), with
    // the 8-chunk groups of odd rows rotated to spread LDS banks
    const int mj = tid >> 3;
    const int msub = tid & 7;

    // out^T[d][r] = sum_c W_UV[d][c] O~[r][c]; B operand column r = lane % 32
    const int j = lane & 31;
    const int b_base = j * 1024 + ((half ^ lat_swz(j)) << 4);
    auto uv_product = [&](int sl) {
        f32x16 part = {};
        const unsigned char* src = stage + sl * kUvRows * 1024;
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) {
            const bf16x8 bv = *reinterpret_cast<const bf16x8*>(src + ((b_base ^ ((ks & 7) << 5)) + (ks >> 3) * 256));
            part = mfma32(wa[ks], bv, part);
        }
        return part;
    };
    auto store_out = [&](const f32x16& acc) {
        const int r = rb * kUvRows + j;
        if (r < R) {
            __bf16* dst = out + ((size_t)r * kHeads + h) * kValue + 32 * wave + 4 * half;
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<bf16x4*>(dst + 8 * g) =
                    to_bf16x4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
        }
    };
    // heads whose attention pass was marked inexact: recompute exactly into
    // staged slot 0 and give those columns its product instead
    auto exact_heads = [&](f32x16& acc) {
        int any = 0;
        for (int row = 0; row < kUvRows; ++row) any |= marked[row];
        if (!any) return;
        __syncthreads();                     // every staged row read
        for (int row = 0; row < kUvRows; ++row) {
            if (!marked[row]) continue;
            exact_mix(a, rb * kUvRows + row, h, xo, xred, xp, xpos);
            for (int c = tid; c < kLatent; c += 256)
                *reinterpret_cast<__bf16*>(stage + uv_pos(row, c)) = (__bf16)xo[c];
            __syncthreads();
        }
        const f32x16 part = uv_product(0);
        if (marked[j]) acc = part;
    };

    if (n_split <= kUvGroup) {
        // Every split fits in LDS at once.  Each wave fetches rows 8w .. 8w+7
        // of every split with plain 16-byte loads (a run of LDS-direct load
        // groups would go one group at a time per wave, as each group's M0
        // must stay put until it lands) and writes them to LDS, two splits
        // at a time.  Order of the loads: the per-split maxima and sums, the
        // first two splits, W_UV (on the first block), the other two splits,
        // so that every wait the compiler places for a register counts only
        // loads issued after it.  The products run split by split as the
        // data lands and are combined with the merge weights in float32 (the
        // product is linear in O~).
        const int rr_m = rb * kUvRows + mj;
        const bool have = rr_m < R && msub < n_split;
        float m0 = -INFINITY, l0 = 0.f;
        if (have) {
            const size_t o = ((size_t)msub * R + rr_m) * kHeads + h;
            l0 = e.l_part[o];
            m0 = e.m_part[o];
        }
        // rows of one split as a buffer (rows past R read zeros, no branch)
        const unsigned row_bytes = kHeads * kLatent * 2;
        const int rows_here = min(R - rb * kUvRows, kUvRows);
        auto load_rows = [&](int sp, u32x4 (&v)[8]) {
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(
                o_ws + (((size_t)sp * R + rb * kUvRows) * kHeads + h) * kLatent, (unsigned)rows_here * row_bytes);
#pragma unroll
            for (int r8 = 0; r8 < 8; ++r8)
                v[r8] = buf_load16(rs, (unsigned)(8 * wave + r8) * row_bytes + 16u * lane);
        };
        auto store_rows = [&](int sp, const u32x4 (&v)[8]) {
#pragma unroll
            for (int r8 = 0; r8 < 8; ++r8) {
                const int jj = 8 * wave + r8;
                *reinterpret_cast<u32x4*>(stage + (sp * kUvRows + jj) * 1024 +
                                          (((lane & ~15) | ((lane & 15) ^ lat_swz(jj))) << 4)) = v[r8];
            }
        };
        f32x16 part[kUvGroup];
        {
            u32x4 v0[8], v1[8];
            load_rows(0, v0);
            if (n_split > 1) load_rows(1, v1);
            if (kLoadW) uv_load_w(w_uv, h, wa);
            store_rows(0, v0);
            if (n_split > 1) store_rows(1, v1);
        }
        barrier_lds();                       // splits 0 and 1 of every wave in LDS
        if (n_split > 2) {
            u32x4 v2[8], v3[8];
            load_rows(2, v2);
            if (n_split > 3) load_rows(3, v3);
            part[0] = uv_product(0);
            part[1] = uv_product(1);
            store_rows(2, v2);
            if (n_split > 3) store_rows(3, v3);
            barrier_lds();                   // splits 2 and 3 in LDS
            part[2] = uv_product(2);
            if (n_split > 3) part[3] = uv_product(3);
        } else {
            part[0] = uv_product(0);
            if (n_split > 1) part[1] = uv_product(1);
        }
        // merge weights: lane msub of row mj holds split msub's (m, l)
        float mloc = -INFINITY, wloc = 0.f;
        int bad = 0;
        if (have) {
            bad = l0 < 0.f;
            if (l0 > 0.f) {
                mloc = m0;
                wloc = l0;
            }
        }
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) {
            const float m2 = __shfl_xor(mloc, o);
            const float w2 = __shfl_xor(wloc, o);
            const float mx = fmaxf(mloc, m2);
            wloc = (wloc > 0.f ? wloc * exp2f(mloc - mx) : 0.f) + (w2 > 0.f ? w2 * exp2f(m2 - mx) : 0.f);
            mloc = mx;
            bad |= __shfl_xor(bad, o);
        }
        const float inv = wloc > 0.f ? 1.f / wloc : 0.f;
        if (msub == 0) marked[mj] = bad;
        if (msub < kUvGroup) s_w[msub][mj] = (have && !bad) ? weight(m0, l0, mloc, inv) : 0.f;
        __syncthreads();
        f32x16 acc = {};
#pragma unroll
        for (int sl = 0; sl < kUvGroup; ++sl) {
            if (sl >= n_split) break;
            const float w = s_w[sl][j];
            if (w != 0.f)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] += w * part[sl][i];
        }
        exact_heads(acc);
        store_out(acc);
        __syncthreads();                     // staging reused by the next block
        return;
    }

    {
        stage_group(rb, 0);
        // per-row maximum, inverse weight sum and inexact flag over all splits;
        // lanes mj*8 .. mj*8+7 share row mj, lane msub takes splits msub + 8i
        {
            const int rr = rb * kUvRows + mj;
            float mloc = -INFINITY, wloc = 0.f, m0 = -INFINITY, l0 = 0.f;
            int bad = 0;
            if (rr < R) {
                for (int sp = msub; sp < n_split; sp += 8) {
                    const size_t o = ((size_t)sp * R + rr) * kHeads + h;
                    const float l = e.l_part[o];
                    const float m = e.m_part[o];
                    if (sp == msub) {
                        m0 = m;
                        l0 = l;
                    }
                    bad |= l < 0.f;
                    const bool ok = l > 0.f;
                    const float mn = ok ? fmaxf(mloc, m) : mloc;
                    wloc = (wloc > 0.f ? wloc * exp2f(mloc - mn) : 0.f) + (ok ? l * exp2f(m - mn) : 0.f);
                    mloc = mn;
                }
            }
#pragma unroll
            for (int o = 1; o < 8; o <<= 1) {
                const float m2 = __shfl_xor(mloc, o);
                const float w2 = __shfl_xor(wloc, o);
                const float mx = fmaxf(mloc, m2);
                wloc = (wloc > 0.f ? wloc * exp2f(mloc - mx) : 0.f) + (w2 > 0.f ? w2 * exp2f(m2 - mx) : 0.f);
                mloc = mx;
                bad |= __shfl_xor(bad, o);
            }
            const float inv = wloc > 0.f ? 1.f / wloc : 0.f;
            if (msub == 0) {
                s_mmax[mj] = mloc;
                s_inv[mj] = inv;
                marked[mj] = bad;
            }
            // weights of the first staged group come from the values at hand; a
            // head marked for exact recomputation takes nothing from its splits
            if (msub < kUvGroup)
                s_w[msub][mj] = (rr < R && msub < n_split && !bad) ? weight(m0, l0, mloc, inv) : 0.f;
        }
        float x[8][8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) x[i][e] = 0.f;

        for (int g0 = 0; g0 < n_split; g0 += kUvGroup) {
            if (g0 > 0) {
                __syncthreads();             // previous group fully read
                stage_group(rb, g0);
                if (tid < kUvGroup * kUvRows) {
                    const int sl = tid >> 5, j = tid & 31;
                    const int rr = rb * kUvRows + j;
                    float w = 0.f;
                    if (rr < R && g0 + sl < n_split) {
                        const size_t o = ((size_t)(g0 + sl) * R + rr) * kHeads + h;
                        w = weight(e.m_part[o], e.l_part[o], s_mmax[j], s_inv[j]);
                    }
                    s_w[sl][j] = w;
                }
            }
            __builtin_amdgcn_s_waitcnt(0);   // own partial rows landed
            __syncthreads();                 // all rows and weights visible
            const int gn = min(kUvGroup, n_split - g0);
            for (int sl = 0; sl < gn; ++sl) {
                const float w = s_w[sl][mj];
                if (w == 0.f) continue;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int pos = (8 * i + msub) ^ ((mj & 1) << 3);
                    const bf16x8 v = *reinterpret_cast<const bf16x8*>(stage + (sl * kUvRows + mj) * 1024 + pos * 16);
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[i][e] += w * (float)v[e];
                }
            }
        }
        __syncthreads();                     // every staged row read
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int pos = (8 * i + msub) ^ ((mj & 1) << 3);
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (__bf16)x[i][e];
            *reinterpret_cast<bf16x8*>(stage + mj * 1024 + pos * 16) = v;
        }
        __syncthreads();
        // heads whose attention pass was marked inexact: recompute exactly
        for (int row = 0; row < kUvRows; ++row) {
            if (!marked[row]) continue;
            exact_mix(a, rb * kUvRows + row, h, xo, xred, xp, xpos);
            for (int c = tid; c < kLatent; c += 256)
                *reinterpret_cast<__bf16*>(stage + uv_pos(row, c)) = (__bf16)xo[c];
            __syncthreads();
        }
        store_out(uv_product(0));
        __syncthreads();                     // staging reused by the next block
    }
}

__global__ __launch_bounds__(256, 1) void uv_bf16(const __bf16* o, const float* m_part, const float* l_part,
                                                  const __bf16* __restrict__ w_uv, int R, int n_split,
                                                  int r_groups, __bf16* __restrict__ out, AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kUvLds];
    const UvEarly early{o, m_part, l_part, R, n_split};
    const int h = blockIdx.x;
    bf16x8 wa[32];
    // With at most kUvGroup splits the first block loads W_UV itself, after
    // its first partial rows; otherwise W_UV is loaded here, once.
    int rb = blockIdx.y;
    if (n_split <= kUvGroup) {
        uv_block<true>(a, early, out, h, rb, wa, lds, w_uv);
        rb += r_groups;
    } else {
        uv_load_w(w_uv, h, wa);
    }
    for (; rb * kUvRows < R; rb += r_groups) uv_block<false>(a, early, out, h, rb, wa, lds, w_uv);
}

}  // namespace

hipError_t launch_absorb_bf16(const void* q_nope, const void* q_pe, const void* w_uk, void* q_out,
                              int R, hipStream_t s) {
    // one workgroup per (head, quarter of c) and eight query blocks: the
    // weight is read once per eight blocks
    const int blocks = (R + 31) / 32;
    const int r_groups = (blocks + 7) / 8;
    hipLaunchKernelGGL(absorb_q_bf16, dim3(kHeads * 4, r_groups), dim3(256), 0, s,
                       static_cast<const __bf16*>(q_nope), static_cast<const __bf16*>(q_pe),
                       static_cast<const __bf16*>(w_uk), static_cast<__bf16*>(q_out), R, r_groups);
    return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
    const int row_groups = (a.R + 7) / 8;
    hipExtLaunchKernelGGL(attn_bf16, dim3(row_groups * 8 * a.n_split), dim3(256), 0, s, start, stop, 0,
                          a.kv, a.pe, a.idx, a.q, a.R, a.T, a.k, a.n_split, a.slots_per_split, a.causal_base,
                          a.cache_rows_per_query, a);
    return hipGetLastError();
}

hipError_t launch_uv_bf16(const AttnArgs& a, const void* w_uv, void* out, hipStream_t s) {
    const int blocks = (a.R + 31) / 32;
    const int r_groups = blocks < 8 ? blocks : 8;
    hipLaunchKernelGGL(uv_bf16, dim3(kHeads, r_groups), dim3(256), 0, s, static_cast<const __bf16*>(a.o),
                       a.m_part, a.l_part, static_cast<const __bf16*>(w_uv), a.R, a.n_split, r_groups,
                       static_cast<__bf16*>(out), a);
    return hipGetLastError();
}

}  // namespace mla
