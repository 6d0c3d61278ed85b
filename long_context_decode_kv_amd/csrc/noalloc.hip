// attn_decode_noalloc: attn_decode for callers that cannot allocate device
// memory. The decode's scratch (the fused merge's ticket counters and the fp32
// split partials) lives in one fixed array per GPU that the library owns for
// the life of the process, instead of a caller-provided workspace.
#include "attn.h"

#include <mutex>
#include <stdio.h>

#include "internal.h"

namespace attn {

// Bytes of the fixed per-GPU scratch array: the counter block and the
// partials of up to 28 MiB (e.g. 32 query rows x 1024 splits).
constexpr size_t kNoAllocScratchBytes = 32u << 20;

namespace {

// The array itself. In host code this name is only a stand-in for the
// symbol: its device address, one per GPU, comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Address of this device's array, looked up on the first call on the device
// with that device current. nullptr (and *err set) on failure.
void* scratch_for_current_device(hipError_t* err) {
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch[dev] = ptr;
    }
    return g_scratch[dev];
}

}  // namespace
}  // namespace attn

extern "C" {

attn_status attn_decode_noalloc(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                                const float* k_scale, const float* v_scale, const int32_t* kv_lens, int B, int Hq,
                                int Hkv, int d, int L_cap, float softmax_scale, int causal, int num_splits,
                                attn_tensor* out, float* lse, void* stream) {
    attn::set_last_error("");
    // The scratch this call needs follows from the split plan: a function of
    // the shapes (and, for num_splits == 0, of the device's CU count).
    if (!k) {
        attn::set_last_error("k: null tensor");
        return ATTN_ERR_INVALID_ARG;
    }
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || L_cap <= 0 || num_splits < 0) {
        attn::set_last_error("sizes must be positive and num_splits >= 0 (B=%d Hq=%d Hkv=%d d=%d L_cap=%d S=%d)", B,
                             Hq, Hkv, d, L_cap, num_splits);
        return ATTN_ERR_INVALID_ARG;
    }
    const int requested =
        num_splits > 0 ? num_splits : attn_decode_auto_splits(B, Hkv, L_cap, k->dtype, kv_lens != nullptr);
    if (requested <= 0) {
        attn::set_last_error("could not query the device for the split plan");
        return ATTN_ERR_HIP;
    }
    const int S = attn_decode_plan(L_cap, requested, nullptr);
    const size_t need = attn_decode_workspace_size(B, Hq, d, S);
    if (need > attn::kNoAllocScratchBytes) {
        attn::set_last_error("attn_decode_noalloc: %d splits of %d query rows need %zu bytes of scratch; the fixed "
                             "array holds %zu",
                             S, B * Hq, need, attn::kNoAllocScratchBytes);
        return ATTN_ERR_WORKSPACE;
    }
    hipError_t e = hipSuccess;
    void* ws = attn::scratch_for_current_device(&e);
    if (!ws) {
        attn::set_last_error("attn_decode_noalloc: no device address for the scratch array: %s",
                             hipGetErrorString(e));
        return ATTN_ERR_HIP;
    }
    // The array keeps what the previous call left in it. When this call takes
    // the fused merge, the counter lines of its (sequence, KV head) groups are
    // cleared first (after validation, before the decode launch, on `stream`).
    int64_t groups = (int64_t)B * Hkv;
    if (groups > attn::kMaxCounterGroups) groups = attn::kMaxCounterGroups;
    const size_t counter_bytes = (size_t)groups * (1 + attn::kMaxTicketBlocks) * attn::kCounterStride * 4;
    return attn::decode_impl(q, k, v, k_scale, v_scale, kv_lens, B, Hq, Hkv, d, L_cap, softmax_scale, causal,
                             num_splits, out, lse, ws, attn::kNoAllocScratchBytes, counter_bytes, stream);
}

}  // extern "C"
