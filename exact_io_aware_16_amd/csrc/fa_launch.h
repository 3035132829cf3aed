// Internal launch interface between the C-ABI layer (fa_api.hip) and the
// kernel files.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <atomic>

namespace fa {

// ---------------------------------------------------------------------------
// Per-device facts and kernel attributes, looked up once per process.  The
// runtime calls behind them (attribute queries, hipFuncSetAttribute) are host
// work that every launch would otherwise repeat.  Devices numbered at or past
// kMaxDevices are served without the cache.
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;

// Compute units and bytes of LDS per compute unit of the current device.
inline hipError_t device_caps(int* ncu, int* lds_per_cu) {
    static std::atomic<int> cu_cache[kMaxDevices];
    static std::atomic<int> lds_cache[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < kMaxDevices;
    if (cached) {
        const int c = cu_cache[dev].load(std::memory_order_relaxed);
        const int l = lds_cache[dev].load(std::memory_order_relaxed);
        if (c > 0 && l > 0) {
            *ncu = c;
            *lds_per_cu = l;
            return hipSuccess;
        }
    }
    int c = 0, l = 0;
    if ((e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&l, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev)) != hipSuccess)
        return e;
    if (cached) {
        cu_cache[dev].store(c, std::memory_order_relaxed);
        lds_cache[dev].store(l, std::memory_order_relaxed);
    }
    *ncu = c;
    *lds_per_cu = l;
    return hipSuccess;
}

// Raise the dynamic-LDS limit of kernel Kern to `bytes` on the current device,
// the first time it is launched there (every instantiation keeps its own mask
// of the devices already set up; a repeat of the call is harmless).
template <auto Kern>
hipError_t ensure_dynamic_lds(int bytes) {
    static std::atomic<unsigned long long> done{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const unsigned long long bit = (dev >= 0 && dev < kMaxDevices) ? (1ull << dev) : 0ull;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kern), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
}

// A paged K/V cache: pools [num_pages][Hkv][page_size][d]; key j of sequence
// b is row j % page_size of page table[b * max_pages + j / page_size] (entries
// are clamped to [0, num_pages)).  page_size is a multiple of 32.
struct PageTable {
    const int* table;
    int page_size, max_pages, num_pages;
};

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, Hq, Hkv, Nq, Nk, d;
    float scale;
    int causal;
    void* stream;
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dO;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    int grad_bf16;
    int B, Hq, Hkv, Nq, Nk, d;
    float scale;
    int causal;
    float* delta;  // workspace: [2][B][Hq][Nq] float32 (D, then lse log2 e for bf16 inputs)
    void* stream;
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const int* seqlens;
    void* o;
    float* lse;
    int B, Hq, Hkv, Nmax, d;
    float scale;
    float* part_o;    // workspace: [slots][rows per slot][d] float32
    float* part_lse;  // workspace: [slots][rows per slot] float32
    int* meta;        // workspace: [B + 1] int32 (stage prefix per sequence)
    void* stream;
    // Query rows per head forming one causal chunk (the last cq rows of the
    // sequence, bottom-right aligned): Hq then counts (head, token) rows, cq
    // consecutive ones per head.  1 for plain decode and non-causal chunks.
    int cq = 1;
    // paged cache (table == nullptr: k and v are [B][Hkv][Nmax][d]); with a
    // table, Nmax is the capacity max_pages * page_size
    PageTable pages{nullptr, 0, 0, 0};
};

hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a, const int* kv_lens, const PageTable* pages = nullptr);
hipError_t launch_bwd_bf16(const BwdArgs& a);
hipError_t launch_bwd_f32(const BwdArgs& a);
hipError_t launch_decode_bf16(const DecodeArgs& a);

// FP8 forward: q, k, v E4M3 codes with per-tensor descales; o bfloat16.
struct Fp8Args {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, Hq, Hkv, Nq, Nk, d;
    float descale_q, descale_k, descale_v, scale;
    int causal;
    void* stream;
};
hipError_t launch_fwd_fp8(const Fp8Args& a);

// Workspace of the decode path: partial results for at most
// (B * Hkv * ceil(g / 32) + kDecodeMaxWaves) slots of min(g, 32) rows each,
// plus B + 1 stage-prefix integers.
constexpr int kDecodeMaxWaves = 2048;
inline size_t decode_workspace_bytes(int B, int Hq, int Hkv, int Nmax, int d) {
    (void)Nmax;
    const int g = Hq / Hkv, nht = (g + 31) / 32, tr = g < 32 ? g : 32;
    const size_t slots = (size_t)B * Hkv * nht + kDecodeMaxWaves;
    return slots * tr * (size_t)(d + 1) * sizeof(float) + ((size_t)B + 1) * sizeof(int);
}
// Points part_o, part_lse and meta of a into the workspace ws.
inline void decode_workspace_layout(DecodeArgs& a, float* ws) {
    const int g = a.Hq / a.Hkv, nht = (g + 31) / 32, tr = g < 32 ? g : 32;
    const size_t rows = ((size_t)a.B * a.Hkv * nht + kDecodeMaxWaves) * tr;
    a.part_o = ws;
    a.part_lse = ws + rows * a.d;
    a.meta = reinterpret_cast<int*>(a.part_lse + rows);
}

}  // namespace fa
