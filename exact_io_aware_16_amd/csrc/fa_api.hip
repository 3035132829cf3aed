// C ABI of libfa (declared in include/fa.h): argument validation, workspace
// sizing and launch.  Every check happens on the host before anything is
// enqueued.  Between calls the library keeps only per-device facts looked up
// once (CU count, LDS size, each kernel's dynamic-LDS attribute, the address
// of fa_decode_noalloc's scratch) and that scratch itself.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "../../include/fa.h"
#include "fa_launch.h"

// Device scratch of fa_decode_noalloc: one copy per device, reserved when the
// library's code object is loaded on that device and held until the process
// ends.  Host code never passes this name to a kernel (on the host it is a
// stand-in, not a device address); scratch_address() looks up the device
// address once per device and every launch uses that.
static __device__ __align__(256) unsigned char scratch[FA_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

// Address of the current device's `scratch`, looked up with
// hipGetSymbolAddress the first time a device is seen (devices numbered at or
// past kMaxDevices are looked up on every call).
hipError_t scratch_address(void** out) {
    static std::atomic<void*> addr[fa::kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < fa::kMaxDevices;
    if (cached) {
        void* p = addr[dev].load(std::memory_order_acquire);
        if (p) {
            *out = p;
            return hipSuccess;
        }
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    if (cached) addr[dev].store(p, std::memory_order_release);
    *out = p;
    return hipSuccess;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

constexpr int64_t kMaxElems = int64_t(1) << 31;

bool too_big(int64_t a, int64_t b, int64_t c, int64_t d) { return a * b * c * d >= kMaxElems; }

// most new tokens per fa_decode_chunk call
constexpr int kMaxChunk = 64;

fa_status_t check_scale(float scale) {
    return (isfinite(scale) && scale > 0.f) ? FA_OK : FA_ERR_ARG;
}

fa_status_t from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }


}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_str(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_NULL_PTR: return "FA_ERR_NULL_PTR: a required pointer is NULL";
        case FA_ERR_SHAPE: return "FA_ERR_SHAPE: invalid sizes (size < 1, Hq % Hkv != 0, causal with Nq > Nk, or tensor too large)";
        case FA_ERR_DTYPE: return "FA_ERR_DTYPE: unknown dtype, or bfloat16 gradients of float32 inputs";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dimension must be 64 or 128";
        case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
        case FA_ERR_HIP: return "FA_ERR_HIP: kernel launch failed";
        case FA_ERR_ARG: return "FA_ERR_ARG: scale must be finite and > 0, pointers 16-byte aligned";
        case FA_ERR_SCRATCH:
            return "FA_ERR_SCRATCH: the shape needs more device scratch than fa_decode_noalloc's fixed buffer holds";
        default: return "unknown fa status";
    }
}

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                   int Nq, int Nk, int d, fa_dtype_t dtype, float scale, int causal, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_PTR;
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (causal && Nq > Nk) return FA_ERR_SHAPE;
    if (too_big(B, Hq, Nq, d) || too_big(B, Hkv, Nk, d)) return FA_ERR_SHAPE;
    if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (check_scale(scale) != FA_OK) return FA_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse)) return FA_ERR_ARG;
    fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal ? 1 : 0, stream};
    return from_hip(dtype == FA_BF16 ? fa::launch_fwd_bf16(a) : fa::launch_fwd_f32(a, nullptr));
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Nq, int d) {
    (void)d;
    if (B < 1 || Hq < 1 || Nq < 1) return 0;
    return 2 * (size_t)B * Hq * Nq * sizeof(float);
}

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                   void* dq, void* dk, void* dv, fa_dtype_t grad_dtype, int B, int Hq, int Hkv, int Nq, int Nk,
                   int d, fa_dtype_t dtype, float scale, int causal, void* workspace, size_t workspace_bytes,
                   void* stream) {
    if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return FA_ERR_NULL_PTR;
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (causal && Nq > Nk) return FA_ERR_SHAPE;
    if (too_big(B, Hq, Nq, d) || too_big(B, Hkv, Nk, d)) return FA_ERR_SHAPE;
    if ((dtype != FA_F32 && dtype != FA_BF16) || (grad_dtype != FA_F32 && grad_dtype != FA_BF16))
        return FA_ERR_DTYPE;
    // float32 inputs produce float32 gradients only
    if (dtype == FA_F32 && grad_dtype != FA_F32) return FA_ERR_DTYPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (check_scale(scale) != FA_OK) return FA_ERR_ARG;
    if (!workspace || workspace_bytes < fa_bwd_workspace_bytes(B, Hq, Nq, d)) return FA_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) || !aligned4(lse) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
        return FA_ERR_ARG;
    fa::BwdArgs a{q, k, v, o, dO, lse, dq, dk, dv, grad_dtype == FA_BF16 ? 1 : 0, B, Hq, Hkv, Nq, Nk, d,
                  scale, causal ? 1 : 0, static_cast<float*>(workspace), stream};
    return from_hip(dtype == FA_BF16 ? fa::launch_bwd_bf16(a) : fa::launch_bwd_f32(a));
}

size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int Nmax, int d) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Nmax < 1 || d < 1 || Hq % Hkv != 0) return 0;
    return fa::decode_workspace_bytes(B, Hq, Hkv, Nmax, d);
}

fa_status_t fa_decode(const void* q, const void* k_cache, const void* v_cache, const int* seqlens, void* o,
                      float* lse, int B, int Hq, int Hkv, int Nmax, int d, fa_dtype_t dtype, float scale,
                      void* workspace, size_t workspace_bytes, void* stream) {
    if (!q || !k_cache || !v_cache || !seqlens || !o || !lse) return FA_ERR_NULL_PTR;
    if (B < 1 || Hq < 1 || Hkv < 1 || Nmax < 1 || d < 1) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (too_big(B, Hq, 1, d) || too_big(B, Hkv, Nmax, d)) return FA_ERR_SHAPE;
    if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (check_scale(scale) != FA_OK) return FA_ERR_ARG;
    if (!workspace || workspace_bytes < fa_decode_workspace_bytes(B, Hq, Hkv, Nmax, d)) return FA_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned4(seqlens) || !aligned16(o) ||
        !aligned4(lse) || !aligned16(workspace))
        return FA_ERR_ARG;
    if (dtype == FA_F32) {
        // float32: the forward kernel with per-sequence key limits (one query row)
        fa::FwdArgs a{q, k_cache, v_cache, o, lse, B, Hq, Hkv, 1, Nmax, d, scale, 0, stream};
        return from_hip(fa::launch_fwd_f32(a, seqlens));
    }
    fa::DecodeArgs a{q, k_cache, v_cache, seqlens, o, lse, B, Hq, Hkv, Nmax, d, scale, nullptr, nullptr,
                     nullptr, stream};
    float* ws = static_cast<float*>(workspace);
    fa::decode_workspace_layout(a, ws);
    return from_hip(fa::launch_decode_bf16(a));
}

fa_status_t fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int* seqlens,
                              void* o, float* lse, int B, int Hq, int Hkv, int Nmax, int d, fa_dtype_t dtype,
                              float scale, void* stream) {
    if (!q || !k_cache || !v_cache || !seqlens || !o || !lse) return FA_ERR_NULL_PTR;
    if (B < 1 || Hq < 1 || Hkv < 1 || Nmax < 1 || d < 1) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (too_big(B, Hq, 1, d) || too_big(B, Hkv, Nmax, d)) return FA_ERR_SHAPE;
    if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (check_scale(scale) != FA_OK) return FA_ERR_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned4(seqlens) || !aligned16(o) ||
        !aligned4(lse))
        return FA_ERR_ARG;
    if (dtype == FA_F32) {
        // float32 runs the forward kernel with per-sequence key limits: no scratch
        fa::FwdArgs a{q, k_cache, v_cache, o, lse, B, Hq, Hkv, 1, Nmax, d, scale, 0, stream};
        return from_hip(fa::launch_fwd_f32(a, seqlens));
    }
    // the same partial results as fa_decode, in the fixed scratch instead of a
    // caller workspace (nothing in it needs to start at zero: each launch
    // writes every slot its combine reads, and discards the others by select)
    if (fa::decode_workspace_bytes(B, Hq, Hkv, Nmax, d) > (size_t)FA_DECODE_NOALLOC_SCRATCH_BYTES)
        return FA_ERR_SCRATCH;
    void* ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return FA_ERR_HIP;
    fa::DecodeArgs a{q, k_cache, v_cache, seqlens, o, lse, B, Hq, Hkv, Nmax, d, scale, nullptr, nullptr,
                     nullptr, stream};
    fa::decode_workspace_layout(a, static_cast<float*>(ws));
    return from_hip(fa::launch_decode_bf16(a));
}

size_t fa_decode_chunk_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nmax, int d) {
    if (Nq < 1 || Nq > kMaxChunk || B < 1 || Hq < 1 || Hkv < 1 || Nmax < 1 || d < 1 || Hq % Hkv != 0) return 0;
    return fa::decode_workspace_bytes(B, Hq * Nq, Hkv, Nmax, d);
}

fa_status_t fa_decode_chunk(const void* q, const void* k_cache, const void* v_cache, const int* seqlens, void* o,
                            float* lse, int B, int Hq, int Hkv, int Nq, int Nmax, int d, fa_dtype_t dtype,
                            float scale, int causal, void* workspace, size_t workspace_bytes, void* stream) {
    if (!q || !k_cache || !v_cache || !seqlens || !o || !lse) return FA_ERR_NULL_PTR;
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nmax < 1 || d < 1) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0 || Nq > kMaxChunk) return FA_ERR_SHAPE;
    if (too_big(B, Hq, Nq, d) || too_big(B, Hkv, Nmax, d)) return FA_ERR_SHAPE;
    if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (check_scale(scale) != FA_OK) return FA_ERR_ARG;
    if (!workspace || workspace_bytes < fa_decode_chunk_workspace_bytes(B, Hq, Hkv, Nq, Nmax, d))
        return FA_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned4(seqlens) || !aligned16(o) ||
        !aligned4(lse) || !aligned16(workspace))
        return FA_ERR_ARG;
    if (dtype == FA_F32) {
        // float32: the forward kernel with per-sequence key limits; its causal
        // offset is taken from each sequence's own length
        fa::FwdArgs a{q, k_cache, v_cache, o, lse, B, Hq, Hkv, Nq, Nmax, d, scale, causal ? 1 : 0, stream};
        return from_hip(fa::launch_fwd_f32(a, seqlens));
    }
    // bfloat16: the streaming decode over the Hq * Nq (head, token) rows; the
    // Nq rows of a head are consecutive in q, o and lse, so a group of K/V
    // head hk is its g * Nq consecutive rows
    fa::DecodeArgs a{q, k_cache, v_cache, seqlens, o, lse, B, Hq * Nq, Hkv, Nmax, d, scale, nullptr, nullptr,
                     nullptr, stream};
    a.cq = causal ? Nq : 1;
    float* ws = static_cast<float*>(workspace);
    fa::decode_workspace_layout(a, ws);
    return from_hip(fa::launch_decode_bf16(a));
}

fa_status_t fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                       int Nq, int Nk, int d, float descale_q, float descale_k, float descale_v, float scale,
                       int causal, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_PTR;
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (causal && Nq > Nk) return FA_ERR_SHAPE;
    if (too_big(B, Hq, Nq, d) || too_big(B, Hkv, Nk, d)) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (check_scale(scale) != FA_OK || check_scale(descale_q) != FA_OK || check_scale(descale_k) != FA_OK ||
        check_scale(descale_v) != FA_OK)
        return FA_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse)) return FA_ERR_ARG;
    fa::Fp8Args a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, descale_q, descale_k, descale_v, scale, causal ? 1 : 0,
                  stream};
    return from_hip(fa::launch_fwd_fp8(a));
}

size_t fa_decode_paged_workspace_bytes(int B, int Hq, int Hkv, int Nq, int d) {
    return fa_decode_chunk_workspace_bytes(B, Hq, Hkv, Nq, 1, d);
}

fa_status_t fa_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int* block_table,
                            const int* seqlens, void* o, float* lse, int B, int Hq, int Hkv, int Nq, int num_pages,
                            int page_size, int max_pages, int d, fa_dtype_t dtype, float scale, int causal,
                            void* workspace, size_t workspace_bytes, void* stream) {
    if (!q || !k_pages || !v_pages || !block_table || !seqlens || !o || !lse) return FA_ERR_NULL_PTR;
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || num_pages < 1 || page_size < 1 || max_pages < 1 || d < 1)
        return FA_ERR_SHAPE;
    if (Hq % Hkv != 0 || Nq > kMaxChunk) return FA_ERR_SHAPE;
    if (too_big(B, Hq, Nq, d) || too_big(num_pages, Hkv, page_size, d) || too_big(max_pages, page_size, 1, 1) ||
        too_big(B, max_pages, 1, 1))
        return FA_ERR_SHAPE;
    if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (page_size % 32 != 0) return FA_ERR_UNSUPPORTED;
    if (check_scale(scale) != FA_OK) return FA_ERR_ARG;
    if (!workspace || workspace_bytes < fa_decode_paged_workspace_bytes(B, Hq, Hkv, Nq, d)) return FA_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned4(block_table) ||
        !aligned4(seqlens) || !aligned16(o) || !aligned4(lse) || !aligned16(workspace))
        return FA_ERR_ARG;
    const fa::PageTable pt{block_table, page_size, max_pages, num_pages};
    const int cap = max_pages * page_size;
    if (dtype == FA_F32) {
        fa::FwdArgs a{q, k_pages, v_pages, o, lse, B, Hq, Hkv, Nq, cap, d, scale, causal ? 1 : 0, stream};
        return from_hip(fa::launch_fwd_f32(a, seqlens, &pt));
    }
    fa::DecodeArgs a{q, k_pages, v_pages, seqlens, o, lse, B, Hq * Nq, Hkv, cap, d, scale, nullptr, nullptr,
                     nullptr, stream};
    a.cq = causal ? Nq : 1;
    a.pages = pt;
    float* ws = static_cast<float*>(workspace);
    fa::decode_workspace_layout(a, ws);
    return from_hip(fa::launch_decode_bf16(a));
}

}  // extern "C"
