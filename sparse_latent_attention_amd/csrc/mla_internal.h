// Internal declarations shared by the host layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

constexpr int kHeads = 128;   // n_heads
constexpr int kLatent = 512;  // kv_lora_rank: width of the cached latent c^KV
constexpr int kRope = 64;     // qk_rope_head_dim: width of the shared rotary key
constexpr int kNope = 128;    // qk_nope_head_dim
constexpr int kValue = 128;   // v_head_dim
constexpr int kQRow = kLatent + kRope;  // 576: absorbed query row [q_c | q_pe]

// Attention work split: a workgroup owns all heads of one query row and one
// split of that row's index list; splits hold whole tiles of kTileRows slots
// and at most kMaxSlotsPerSplit slots.
constexpr int kTileRows = 32;
constexpr int kMaxSlotsPerSplit = 2048;
// Largest cache length.  Gathers address one query's latent cache with 32-bit
// byte offsets against a buffer descriptor that covers T KiB plus a 3 KiB
// prefix; an empty slot carries the offset 2^31, which must lie past that
// range for every instruction offset: T*1024 + 3072 <= 2^31.
constexpr int kMaxT = (1 << 21) - 4;

// Workspace carve-up, shared by the size query and the launchers.
struct Workspace {
    size_t q_off, q_bytes;        // absorbed queries [R, 128, 576] in the call dtype
    size_t o_off, o_bytes;        // mixed latent per split [n_split, R, 128, 512]
    size_t ml_off, ml_bytes;      // per split reference max / probability sum [n_split, R, 128] x2 (f32)
    size_t stats_off;             // diagnostics of the call: int32 [0] rerun splits, [1] reserved (0)
    size_t total;
    int n_split;                  // splits of each row's index list
    int slots_per_split;          // index-list slots per split (multiple of kTileRows)
};

Workspace plan_workspace(int rows, int k, int dtype);

// Host-side argument checks of mla_sparse_decode (everything but the
// workspace); returns MLA_OK (0) or the error code, touching no device.
int check_decode_args(const void* q_nope, const void* q_pe, const void* kv_cache,
                      const void* pe_cache, const int32_t* topk_idx, const void* w_uk,
                      const void* w_uv, const void* out, int B, int T, int ld_T, int k,
                      float softmax_scale, int dtype);

struct AttnArgs {
    const void* q;          // [R, 128, 576] absorbed queries
    const void* kv;         // latent cache base
    const void* pe;         // rotary cache base
    const int32_t* idx;     // [R, k]
    long long cache_rows_per_query;  // cache row stride between queries (0 = shared cache)
    int R, T, k;
    int causal_base;        // -1: no causal bound; else query r sees positions <= causal_base + r
    float scale_log2;       // softmax_scale * log2(e)
    int n_split, slots_per_split;
    void* o;                // see Workspace::o
    float* m_part;          // [n_split, R, 128]
    float* l_part;          // [n_split, R, 128]
    int* stats;             // diagnostics (see Workspace::stats_off), zeroed before the attention kernel
};

// Launchers (return hipSuccess or the launch error).  The attention launchers
// take optional start and stop events, which the kernel's dispatch itself
// timestamps (hipExtLaunchKernel): the interval is the kernel's own duration.
// The absorb launchers also zero the call's diagnostics (`stats`), which the
// attention kernel that follows them on the stream then counts into.
hipError_t launch_absorb_bf16(const void* q_nope, const void* q_pe, const void* w_uk, void* q_out,
                              int R, int* stats, hipStream_t s);
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s, hipEvent_t start = nullptr,
                            hipEvent_t stop = nullptr);
hipError_t launch_uv_bf16(const AttnArgs& a, const void* w_uv, void* out, hipStream_t s);


hipError_t launch_absorb_f32(const void* q_nope, const void* q_pe, const void* w_uk, void* q_out,
                             int R, int* stats, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s, hipEvent_t start = nullptr,
                           hipEvent_t stop = nullptr);
hipError_t launch_uv_f32(const float* o_part, const float* m_part, const float* l_part,
                         const void* w_uv, void* out, int R, int n_split, hipStream_t s);

// Explicit-form sparse prefill (mla_sparse_prefill_explicit): workspace =
// up-projected keys/values [Tv, 128, 256] bf16, then the selection bitmap
// [S, words] (32 positions per word), Tv = min(start_pos + S, T).
struct ExplicitPlan {
    int Tv, words;
    size_t up_bytes, bm_off, total;
};
ExplicitPlan plan_explicit(int S, int T, int start_pos);
hipError_t launch_explicit_prefill(const void* q_nope, const void* q_pe, const void* kv, const void* pe,
                                   const int32_t* idx, const void* w_uk, const void* w_uv, void* out, int S, int k,
                                   int start_pos, float scale_log2, const ExplicitPlan& p, void* ws, hipStream_t s);

// FP8 wkv_b dequantisation (mla_wkv_b_dequant)
hipError_t launch_wkv_b_dequant(const void* codes, const float* scales, void* w_uk, void* w_uv, hipStream_t s);

// Output projection (mla_output_projection): [B, 16384] . [7168, 16384]^T.
constexpr int kProjIn = kHeads * kValue;   // 16,384 joined head outputs
constexpr int kProjOut = 7168;             // model width
size_t project_workspace_bytes(int B, bool bf16);
hipError_t launch_project(const void* o, const void* w_o, void* out, int B, bool bf16, void* ws, hipStream_t s);

// Cache append (mla_cache_append): one wave per new position.
hipError_t launch_cache_append(const void* kv_a_out, const void* norm_weight, const float* cos_sin, void* kv_cache,
                               void* pe_cache, int B, int S, int start_pos, int ld_T, float eps, bool bf16,
                               hipStream_t s);

hipError_t launch_validate(const int32_t* idx, int rows, int k, int T, int allow_pad, int* flag,
                           hipStream_t s);

}  // namespace mla
