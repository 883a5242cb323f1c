// Host side of the C ABI declared in include/mla_sparse.h: argument checks,
// workspace planning and the launch sequence (absorb W_UK -> attention ->
// merge + absorb W_UV), all asynchronous on the caller's stream.
#include "mla_sparse.h"

#include <climits>
#include <cmath>

#include "mla_internal.h"

namespace mla {
namespace {

constexpr size_t kAlign = 256;
constexpr int kTargetGroups = 256;   // workgroups that fill the 256 compute units once

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

hipEvent_t g_attn_begin = nullptr;
hipEvent_t g_attn_end = nullptr;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

Workspace plan_workspace(int rows, int k, int dtype) {
    Workspace w{};
    const size_t esize = dtype == MLA_BF16 ? 2 : 4;
    // Split each index list so that about kTargetGroups workgroups run, with
    // whole 32-row tiles per split and at most kMaxSlotsPerSplit slots each.
    const int max_split = (k + kTileRows - 1) / kTileRows;
    const int min_split = (k + kMaxSlotsPerSplit - 1) / kMaxSlotsPerSplit;
    int n = (kTargetGroups + rows - 1) / rows;
    if (n > max_split) n = max_split;
    if (n < min_split) n = min_split;
    if (n < 1) n = 1;
    int per = (k + n - 1) / n;
    per = (per + kTileRows - 1) / kTileRows * kTileRows;
    n = (k + per - 1) / per;
    w.n_split = n;
    w.slots_per_split = per;

    const size_t R = (size_t)rows;
    w.q_off = 0;
    w.q_bytes = R * kHeads * kQRow * esize;
    w.o_off = round_up(w.q_off + w.q_bytes, kAlign);
    // bf16: per split, the unnormalised mix in bf16 + the reference maximum and
    // the sum of weights against it; f32: per split, the unnormalised mix in
    // f32 + running max and sum.
    const bool bf16 = dtype == MLA_BF16;
    w.o_bytes = (size_t)n * R * kHeads * kLatent * (bf16 ? 2 : 4);
    w.ml_off = round_up(w.o_off + w.o_bytes, kAlign);
    w.ml_bytes = 2 * (size_t)n * R * kHeads * 4;
    w.stats_off = round_up(w.ml_off + w.ml_bytes, kAlign);
    w.total = w.stats_off + kAlign;
    return w;
}

namespace {

mla_status run(const void* q_nope, const void* q_pe, const void* kv_cache, const void* pe_cache,
               const int32_t* idx, const void* w_uk, const void* w_uv, void* out, int R, int T,
               long long cache_rows_per_query, int k, int causal_base, float scale, int dtype,
               void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const Workspace w = plan_workspace(R, k, dtype);
    if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0 ||
        workspace_bytes < w.total)
        return MLA_ERR_WORKSPACE;

    unsigned char* ws = static_cast<unsigned char*>(workspace);
    AttnArgs a{};
    a.q = ws + w.q_off;
    a.kv = kv_cache;
    a.pe = pe_cache;
    a.idx = idx;
    a.cache_rows_per_query = cache_rows_per_query;
    a.R = R;
    a.T = T;
    a.k = k;
    a.causal_base = causal_base;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.n_split = w.n_split;
    a.slots_per_split = w.slots_per_split;
    a.o = ws + w.o_off;
    a.m_part = reinterpret_cast<float*>(ws + w.ml_off);
    a.l_part = reinterpret_cast<float*>(ws + w.ml_off) + (size_t)w.n_split * R * kHeads;
    a.stats = reinterpret_cast<int*>(ws + w.stats_off);

    hipError_t e;
    if (dtype == MLA_BF16)
        e = launch_absorb_bf16(q_nope, q_pe, w_uk, ws + w.q_off, R, a.stats, stream);
    else
        e = launch_absorb_f32(q_nope, q_pe, w_uk, ws + w.q_off, R, a.stats, stream);
    if (e != hipSuccess) return MLA_ERR_HIP;

    hipEvent_t eb = g_attn_begin, ee = g_attn_end;
    g_attn_begin = g_attn_end = nullptr;
    e = dtype == MLA_BF16 ? launch_attn_bf16(a, stream, eb, ee) : launch_attn_f32(a, stream, eb, ee);
    if (e != hipSuccess) return MLA_ERR_HIP;

    if (dtype == MLA_BF16)
        e = launch_uv_bf16(a, w_uv, out, stream);
    else
        e = launch_uv_f32(static_cast<const float*>(a.o), a.m_part, a.l_part, w_uv, out, R,
                          w.n_split, stream);
    return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

bool dtype_ok(int dtype) { return dtype == MLA_F32 || dtype == MLA_BF16; }

}  // namespace

int check_decode_args(const void* q_nope, const void* q_pe, const void* kv_cache,
                      const void* pe_cache, const int32_t* topk_idx, const void* w_uk,
                      const void* w_uv, const void* out, int B, int T, int ld_T, int k,
                      float softmax_scale, int dtype) {
    if (!q_nope || !q_pe || !kv_cache || !pe_cache || !topk_idx || !w_uk || !w_uv || !out)
        return MLA_ERR_NULL;
    if (!dtype_ok(dtype)) return MLA_ERR_DTYPE;
    if (B < 1 || T < 1 || T > kMaxT || k < 1 || k > T || ld_T < T) return MLA_ERR_SHAPE;
    if (dtype == MLA_F32 && B > 65535) return MLA_ERR_SHAPE;
    if (!std::isfinite(softmax_scale)) return MLA_ERR_SHAPE;
    if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(kv_cache) || !aligned16(pe_cache) ||
        !aligned16(topk_idx) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(out))
        return MLA_ERR_ALIGN;
    return MLA_OK;
}

}  // namespace mla

using namespace mla;

extern "C" {

const char* mla_status_string(int s) {
    switch (s) {
        case MLA_OK: return "MLA_OK";
        case MLA_ERR_NULL: return "MLA_ERR_NULL: required pointer is NULL";
        case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: size out of range";
        case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN: tensor pointer not 16-byte aligned";
        case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: unknown dtype";
        case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing, misaligned or too small";
        case MLA_ERR_INDEX: return "MLA_ERR_INDEX: invalid index list";
        case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime or launch failure";
        default: return "MLA_ERR_UNKNOWN";
    }
}

int mla_abi_version(void) { return 3; }

size_t mla_sparse_decode_workspace_size(int B, int T, int k, int dtype) {
    if (!dtype_ok(dtype) || B < 1 || T < 1 || T > kMaxT || k < 1 || k > T) return 0;
    return plan_workspace(B, k, dtype).total;
}

size_t mla_sparse_prefill_chunk_workspace_size(int S, int T, int k, int dtype) {
    if (!dtype_ok(dtype) || S < 1 || T < 1 || T > kMaxT || k < 1) return 0;
    return plan_workspace(S, k, dtype).total;
}

mla_status mla_sparse_decode(const void* q_nope, const void* q_pe, const void* kv_cache,
                             const void* pe_cache, const int32_t* topk_idx, const void* w_uk,
                             const void* w_uv, void* out, int B, int T, int ld_T, int k,
                             float softmax_scale, int dtype, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
    const int st = check_decode_args(q_nope, q_pe, kv_cache, pe_cache, topk_idx, w_uk, w_uv, out, B,
                                     T, ld_T, k, softmax_scale, dtype);
    if (st != MLA_OK) return static_cast<mla_status>(st);
    return run(q_nope, q_pe, kv_cache, pe_cache, topk_idx, w_uk, w_uv, out, B, T, ld_T, k, -1,
               softmax_scale, dtype, workspace, workspace_bytes, stream);
}

mla_status mla_sparse_prefill_chunk(const void* q_nope, const void* q_pe, const void* kv_cache,
                                    const void* pe_cache, const int32_t* topk_idx, const void* w_uk,
                                    const void* w_uv, void* out, int S, int T, int k, int start_pos,
                                    float softmax_scale, int dtype, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    if (!q_nope || !q_pe || !kv_cache || !pe_cache || !topk_idx || !w_uk || !w_uv || !out)
        return MLA_ERR_NULL;
    if (!dtype_ok(dtype)) return MLA_ERR_DTYPE;
    if (S < 1 || T < 1 || T > kMaxT || k < 1 || start_pos < 0 || (long long)start_pos + S > T)
        return MLA_ERR_SHAPE;
    if (dtype == MLA_F32 && S > 65535) return MLA_ERR_SHAPE;
    if (!std::isfinite(softmax_scale)) return MLA_ERR_SHAPE;
    if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(kv_cache) || !aligned16(pe_cache) ||
        !aligned16(topk_idx) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(out))
        return MLA_ERR_ALIGN;
    return run(q_nope, q_pe, kv_cache, pe_cache, topk_idx, w_uk, w_uv, out, S, T, 0, k, start_pos,
               softmax_scale, dtype, workspace, workspace_bytes, stream);
}

mla_status mla_validate_indices(const int32_t* idx, int rows, int k, int T, int allow_pad,
                                int* d_flag, hipStream_t stream) {
    if (!idx || !d_flag) return MLA_ERR_NULL;
    if (rows < 1 || k < 1 || T < 1) return MLA_ERR_SHAPE;
    if (!aligned16(idx) || (reinterpret_cast<uintptr_t>(d_flag) & 3u)) return MLA_ERR_ALIGN;
    return launch_validate(idx, rows, k, T, allow_pad, d_flag, stream) == hipSuccess ? MLA_OK
                                                                                       : MLA_ERR_HIP;
}

mla_status mla_cache_append(const void* kv_a_out, const void* norm_weight, const float* cos_sin, void* kv_cache,
                            void* pe_cache, int B, int S, int start_pos, int ld_T, float eps, int dtype,
                            hipStream_t stream) {
    if (!kv_a_out || !norm_weight || !cos_sin || !kv_cache || !pe_cache) return MLA_ERR_NULL;
    if (!dtype_ok(dtype)) return MLA_ERR_DTYPE;
    if (B < 1 || S < 1 || start_pos < 0 || ld_T < 1 || (long long)start_pos + S > ld_T) return MLA_ERR_SHAPE;
    if (!std::isfinite(eps) || eps < 0.f) return MLA_ERR_SHAPE;
    if (!aligned16(kv_a_out) || !aligned16(norm_weight) || !aligned16(cos_sin) || !aligned16(kv_cache) ||
        !aligned16(pe_cache))
        return MLA_ERR_ALIGN;
    return launch_cache_append(kv_a_out, norm_weight, cos_sin, kv_cache, pe_cache, B, S, start_pos, ld_T, eps,
                               dtype == MLA_BF16, stream) == hipSuccess
               ? MLA_OK
               : MLA_ERR_HIP;
}

size_t mla_sparse_prefill_explicit_workspace_size(int S, int T, int k, int start_pos, int dtype) {
    if (dtype != MLA_BF16 || S < 1 || T < 1 || T > kMaxT || k < 1 || start_pos < 0 ||
        (long long)start_pos + S > T)
        return 0;
    return plan_explicit(S, T, start_pos).total;
}

mla_status mla_sparse_prefill_explicit(const void* q_nope, const void* q_pe, const void* kv_cache,
                                       const void* pe_cache, const int32_t* topk_idx, const void* w_uk,
                                       const void* w_uv, void* out, int S, int T, int k, int start_pos,
                                       float softmax_scale, int dtype, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
    if (!q_nope || !q_pe || !kv_cache || !pe_cache || !topk_idx || !w_uk || !w_uv || !out) return MLA_ERR_NULL;
    if (dtype != MLA_BF16) return MLA_ERR_DTYPE;   // bf16 only
    if (S < 1 || T < 1 || T > kMaxT || k < 1 || start_pos < 0 || (long long)start_pos + S > T)
        return MLA_ERR_SHAPE;
    if (!std::isfinite(softmax_scale)) return MLA_ERR_SHAPE;
    if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(kv_cache) || !aligned16(pe_cache) ||
        !aligned16(topk_idx) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(out))
        return MLA_ERR_ALIGN;
    const ExplicitPlan p = plan_explicit(S, T, start_pos);
    if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0 || workspace_bytes < p.total)
        return MLA_ERR_WORKSPACE;
    return launch_explicit_prefill(q_nope, q_pe, kv_cache, pe_cache, topk_idx, w_uk, w_uv, out, S, k, start_pos,
                                   softmax_scale * 1.4426950408889634f, p, workspace, stream) == hipSuccess
               ? MLA_OK
               : MLA_ERR_HIP;
}

mla_status mla_wkv_b_dequant(const void* codes, const float* scales, void* w_uk, void* w_uv, hipStream_t stream) {
    if (!codes || !scales || !w_uk || !w_uv) return MLA_ERR_NULL;
    if (!aligned16(codes) || (reinterpret_cast<uintptr_t>(scales) & 3u) != 0 || !aligned16(w_uk) || !aligned16(w_uv))
        return MLA_ERR_ALIGN;
    return launch_wkv_b_dequant(codes, scales, w_uk, w_uv, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

size_t mla_output_projection_workspace_size(int B, int dtype) {
    if (!dtype_ok(dtype) || B < 1 || (long long)B * kProjOut > 0x7fffffffLL) return 0;
    return project_workspace_bytes(B, dtype == MLA_BF16);
}

mla_status mla_output_projection(const void* o, const void* w_o, void* out, int B, int dtype, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    if (!o || !w_o || !out) return MLA_ERR_NULL;
    if (!dtype_ok(dtype)) return MLA_ERR_DTYPE;
    if (B < 1 || (long long)B * kProjOut > 0x7fffffffLL) return MLA_ERR_SHAPE;
    if (!aligned16(o) || !aligned16(w_o) || !aligned16(out)) return MLA_ERR_ALIGN;
    const size_t need = project_workspace_bytes(B, dtype == MLA_BF16);
    if (need > 0 && (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0 ||
                     workspace_bytes < need))
        return MLA_ERR_WORKSPACE;
    return launch_project(o, w_o, out, B, dtype == MLA_BF16, workspace, stream) == hipSuccess ? MLA_OK
                                                                                               : MLA_ERR_HIP;
}

mla_status mla_read_diagnostics(const void* workspace, int rows, int k, int dtype, int* d_out,
                                hipStream_t stream) {
    if (!workspace || !d_out) return MLA_ERR_NULL;
    if (!dtype_ok(dtype)) return MLA_ERR_DTYPE;
    if (rows < 1 || k < 1) return MLA_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(d_out) & 3u) != 0) return MLA_ERR_ALIGN;
    const Workspace w = plan_workspace(rows, k, dtype);
    const unsigned char* src = static_cast<const unsigned char*>(workspace) + w.stats_off;
    return hipMemcpyAsync(d_out, src, 2 * sizeof(int), hipMemcpyDeviceToDevice, stream) == hipSuccess
               ? MLA_OK
               : MLA_ERR_HIP;
}

mla_status mla_set_attention_events(hipEvent_t begin, hipEvent_t end) {
    if ((begin == nullptr) != (end == nullptr)) return MLA_ERR_NULL;
    g_attn_begin = begin;
    g_attn_end = end;
    return MLA_OK;
}

}  // extern "C"
