// Allocation-free decode: the same call as mla_sparse_decode, with its
// workspace in a fixed device array of this library instead of caller memory,
// for callers that cannot allocate (code under graph capture, serving loops,
// harnesses that forbid allocation).
#include <mutex>

#include "mla_internal.h"
#include "mla_sparse.h"

namespace mla {
namespace {

// The array is a device symbol: in host code its name is a host-side stand-in,
// never a device address.  Host code only ever uses the per-device address
// that hipGetSymbolAddress returns for it.
static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of `scratch` on the current device, looked up once per device with
// that device current.
mla_status scratch_on_current_device(void** ptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MLA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MLA_OK;
}

}  // namespace
}  // namespace mla

extern "C" mla_status mla_sparse_decode_noalloc(const void* q_nope, const void* q_pe,
                                                const void* kv_cache, const void* pe_cache,
                                                const int32_t* topk_idx, const void* w_uk,
                                                const void* w_uv, void* out, int B, int T, int ld_T,
                                                int k, float softmax_scale, int dtype,
                                                hipStream_t stream) {
    using namespace mla;
    const int st = check_decode_args(q_nope, q_pe, kv_cache, pe_cache, topk_idx, w_uk, w_uv, out, B,
                                     T, ld_T, k, softmax_scale, dtype);
    if (st != MLA_OK) return static_cast<mla_status>(st);
    if (plan_workspace(B, k, dtype).total > (size_t)MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
    void* ws = nullptr;
    const mla_status s = scratch_on_current_device(&ws);
    if (s != MLA_OK) return s;
    return mla_sparse_decode(q_nope, q_pe, kv_cache, pe_cache, topk_idx, w_uk, w_uv, out, B, T, ld_T, k,
                             softmax_scale, dtype, ws, (size_t)MLA_NOALLOC_SCRATCH_BYTES, stream);
}
