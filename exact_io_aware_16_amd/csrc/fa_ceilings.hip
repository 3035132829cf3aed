// Measured ceilings of the GPU the attention kernels run on (libfa_ceilings):
// the throughput of the bf16 matrix-core instruction every bf16 kernel is
// built on, HBM read bandwidth, LDS read bandwidth for the two read forms the
// kernels use (16-byte row reads and 8-byte transposing reads), and the core
// clock the chip holds while its matrix cores are busy.  The attention
// kernels' rooflines are stated against the published peaks; these numbers
// say how much of each peak this part, at the clock it actually runs, can
// deliver to a kernel at all.  Declared in include/fa_ceilings.h.
#include "fa_device.h"
#include "../../include/fa_ceilings.h"

namespace fa {
namespace {

// core-clock cycle counter (s_memtime) and constant-rate counter (s_memrealtime)
__device__ __forceinline__ unsigned long long core_cycles() { return __builtin_readcyclecounter(); }
__device__ __forceinline__ unsigned long long wall_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// Every wave runs `iters` rounds of 4 independent v_mfma_f32_32x32x16_bf16
// (4 accumulators, so each chain's next product issues 4 products later, past
// the instruction's latency).  Lane 0 of each wave records its core-cycle and
// wall-tick counters around the loop; the accumulators are summed into sink
// so the products cannot be removed.
__global__ __launch_bounds__(256) void ceil_mfma_kernel(float* __restrict__ sink,
                                                        unsigned long long* __restrict__ stamps, int iters) {
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)((lane + i) & 7));
        b[i] = (__bf16)(0.002f * (float)((lane * 3 + i) & 7));
    }
    f32x16 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = zero16();
    const unsigned long long c0 = core_cycles(), w0 = wall_ticks();
#pragma unroll 4
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = mfma32x32x16(a, b, acc[u]);
    }
    // the counters read after the last product has completed (its result is used)
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[u][i];
    const unsigned long long c1 = core_cycles(), w1 = wall_ticks();
    s += __shfl_xor(s, 32, 64);
    if (lane == 0) {
        sink[wave] = s;
        stamps[wave * 4 + 0] = c0;
        stamps[wave * 4 + 1] = c1;
        stamps[wave * 4 + 2] = w0;
        stamps[wave * 4 + 3] = w1;
    }
}

// Streaming read of n16 16-byte words: each lane reads U consecutive-stride
// words per step (U loads in flight), grid-stride.  The words are folded with
// xor; the result is stored only if it equals a value the caller never
// plants, so the kernel writes nothing in practice and its time is the read
// alone.
template <int U>
__global__ __launch_bounds__(256) void ceil_read_kernel(const u32x4* __restrict__ buf, long long n16,
                                                        u32x4* __restrict__ sink, uint32_t never) {
    const long long stride = (long long)gridDim.x * 256;
    long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= x[u];
    }
    for (; i < n16; i += stride) acc ^= buf[i];
    if (acc[0] == never && acc[1] == never) sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

// Streaming read through direct-to-LDS loads, the form the decode streams
// its cache with: one-wave workgroups, each reading its contiguous share of
// the buffer in 1 KB instructions (64 lanes x 16 B) into a ring of NS stages
// of L instructions, keeping at most NS - 1 stages in flight.  POL is the
// cache-policy operand (0 default, 2 non-temporal).
template <int L, int NS, int POL>
__global__ __launch_bounds__(64) void ceil_read_lds_kernel(const u32x4* __restrict__ buf, long long units_per_wave) {
    extern __shared__ __align__(16) u32x4 ring[];
    const int lane = threadIdx.x;
    const u32x4* src = buf + (long long)blockIdx.x * units_per_wave * 64 + lane;
    const long long nst = units_per_wave / L;
    for (long long k = 0; k < nst; ++k) {
        u32x4* dst = ring + (int)(k % NS) * L * 64;
#pragma unroll
        for (int i = 0; i < L; ++i)
            __builtin_amdgcn_global_load_lds(src + (k * L + i) * 64, (__attribute__((address_space(3))) void*)(dst + i * 64),
                                             16, 0, POL);
        wait_vmcnt<(NS - 1) * L>();
    }
    wait_vmcnt<0>();
}

// LDS read bandwidth.  Each workgroup fills 64 KB of LDS, then every wave
// reads it `iters` times over: mode 0 with 16-byte reads (ds_read_b128, 64
// lanes x 16 B = 1 KB per instruction, consecutive lanes on consecutive 16-byte
// slots), mode 1 with 8-byte transposing reads (ds_read_b64_tr_b16, 512 B per
// instruction, the lane addressing of the attention kernels' V^T fragments:
// 4 rows x 4 chunks per 16-lane group of a 256-byte-row tile).  Four reads are
// in flight per step; their results are folded with xor.
constexpr int kLdsBytes = 65536;

__global__ __launch_bounds__(256) void ceil_lds_kernel(uint32_t* __restrict__ sink,
                                                       unsigned long long* __restrict__ stamps, int mode,
                                                       int iters) {
    extern __shared__ __align__(16) uint16_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < kLdsBytes / 16; i += 256)
        reinterpret_cast<u32x4*>(lds)[i] = u32x4{(uint32_t)i, (uint32_t)i * 3u, 7u, 9u};
    __syncthreads();
    const unsigned long long c0 = core_cycles(), w0 = wall_ticks();
    u32x4 acc = {0u, 0u, 0u, 0u};
    // The read address passes through an empty asm statement every step, so
    // the compiler cannot see that a window repeats and merge or drop reads
    // (the data is folded with xor, where equal words would cancel).
    if (mode == 0) {
        for (int it = 0; it < iters; ++it) {
            // 4 KB of consecutive slots per step, a different window every step
            int base = ((it * 4 + wave) * 4096) & (kLdsBytes - 1);
            asm volatile("" : "+v"(base));
#pragma unroll
            for (int u = 0; u < 4; ++u)
                acc ^= *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(lds) +
                                                       ((base + u * 1024 + lane * 16) & (kLdsBytes - 1)));
        }
    } else if (mode == 2) {
        for (int it = 0; it < iters; ++it) {
            // 2 KB of consecutive 8-byte slots per step
            int base = ((it * 4 + wave) * 2048) & (kLdsBytes - 1);
            asm volatile("" : "+v"(base));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const u32x2 w = *reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(lds) +
                                                                ((base + u * 512 + lane * 8) & (kLdsBytes - 1)));
                acc[0] ^= w[0];
                acc[1] ^= w[1];
            }
        }
    } else {
        // mode 1: the kernels' swizzled tile; mode 3: the same reads of an
        // unswizzled tile (chunk c of row r at slot c)
        const int t = lane & 15;
        for (int it = 0; it < iters; ++it) {
            // a 32-row x 128-column bf16 tile (8 KB, rows of 256 B) per step;
            // the four reads are the two halves of the fragments at
            // (k0, c0) = (0, 0) and (16, 32)
            int tile = ((it * 4 + wave) * 4096) & (kLdsBytes / 2 - 1);
            asm volatile("" : "+v"(tile));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int k0 = (u >> 1) * 16, c0 = (u >> 1) * 32;
                const int r = k0 + (lane >> 5) * 4 + (t >> 2) + 8 * (u & 1);
                const int c = c0 + ((lane >> 4) & 1) * 16 + (t & 3) * 4;
                const int e = mode == 1 ? swz_off<128>(r, c >> 3) + (c & 7) : r * 128 + c;
                const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (__attribute__((address_space(3))) bf16x4*)(lds + tile + e));
                const u32x2 w = __builtin_bit_cast(u32x2, v);
                acc[0] ^= w[0];
                acc[1] ^= w[1];
            }
        }
    }
    const unsigned long long c1 = core_cycles(), w1 = wall_ticks();
    const uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (r == 0xFFFFFFFFu) sink[blockIdx.x * 256 + tid] = r;
    if (lane == 0) {
        const int gw = blockIdx.x * 4 + wave;
        stamps[gw * 4 + 0] = c0;
        stamps[gw * 4 + 1] = c1;
        stamps[gw * 4 + 2] = w0;
        stamps[gw * 4 + 3] = w1;
    }
}

}  // namespace
}  // namespace fa

namespace fa {
namespace {
template <int L, int NS>
hipError_t launch_read_lds(const u32x4* b, long long upw, int workgroups, int nt, hipStream_t st) {
    const int lds = L * NS * 1024;
    if (nt) {
        constexpr auto kern = ceil_read_lds_kernel<L, NS, 2>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(workgroups), dim3(64), lds, st, b, upw);
    } else {
        constexpr auto kern = ceil_read_lds_kernel<L, NS, 0>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(workgroups), dim3(64), lds, st, b, upw);
    }
    return hipGetLastError();
}
template <int L>
hipError_t launch_read_lds_l(const u32x4* b, long long upw, int workgroups, int stages, int nt, hipStream_t st) {
    if (stages == 2) return launch_read_lds<L, 2>(b, upw, workgroups, nt, st);
    if (stages == 3) return launch_read_lds<L, 3>(b, upw, workgroups, nt, st);
    return launch_read_lds<L, 4>(b, upw, workgroups, nt, st);
}
}  // namespace
}  // namespace fa

extern "C" {

int fa_ceil_device(int* ncu, int* wall_clock_khz, int* peak_clock_khz) {
    if (!ncu || !wall_clock_khz || !peak_clock_khz) return (int)hipErrorInvalidValue;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(wall_clock_khz, hipDeviceAttributeWallClockRate, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(peak_clock_khz, hipDeviceAttributeClockRate, dev);
    return (int)e;
}

int fa_ceil_mfma_bf16(float* sink, unsigned long long* stamps, int workgroups, int iters, void* stream) {
    if (!sink || !stamps || workgroups < 1 || iters < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(fa::ceil_mfma_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, sink, stamps,
                       iters);
    return (int)hipGetLastError();
}

int fa_ceil_hbm_read(const void* buf, size_t bytes, void* sink, int workgroups, int loads_in_flight,
                     void* stream) {
    if (!buf || !sink || bytes < 16 || (bytes & 15) || workgroups < 1 ||
        (loads_in_flight != 4 && loads_in_flight != 8 && loads_in_flight != 16) ||
        (reinterpret_cast<uintptr_t>(buf) & 15) || (reinterpret_cast<uintptr_t>(sink) & 15))
        return (int)hipErrorInvalidValue;
    const auto* b = static_cast<const fa::u32x4*>(buf);
    auto* k = static_cast<fa::u32x4*>(sink);
    const long long n16 = (long long)(bytes / 16);
    const hipStream_t st = (hipStream_t)stream;
    if (loads_in_flight == 4)
        hipLaunchKernelGGL(fa::ceil_read_kernel<4>, dim3(workgroups), dim3(256), 0, st, b, n16, k, 0x9E3779B9u);
    else if (loads_in_flight == 8)
        hipLaunchKernelGGL(fa::ceil_read_kernel<8>, dim3(workgroups), dim3(256), 0, st, b, n16, k, 0x9E3779B9u);
    else
        hipLaunchKernelGGL(fa::ceil_read_kernel<16>, dim3(workgroups), dim3(256), 0, st, b, n16, k, 0x9E3779B9u);
    return (int)hipGetLastError();
}

long long fa_ceil_hbm_read_lds_bytes(size_t bytes, int workgroups, int stage_kb) {
    if (workgroups < 1 || (stage_kb != 4 && stage_kb != 8 && stage_kb != 16)) return 0;
    const long long upw = (long long)(bytes / 1024) / workgroups / stage_kb * stage_kb;
    return upw * 1024 * workgroups;
}

int fa_ceil_hbm_read_lds(const void* buf, size_t bytes, int workgroups, int stage_kb, int stages, int nontemporal,
                         void* stream) {
    if (!buf || (reinterpret_cast<uintptr_t>(buf) & 15) || workgroups < 1 ||
        (stage_kb != 4 && stage_kb != 8 && stage_kb != 16) || stages < 2 || stages > 4 ||
        (nontemporal != 0 && nontemporal != 1))
        return (int)hipErrorInvalidValue;
    const long long upw = (long long)(bytes / 1024) / workgroups / stage_kb * stage_kb;
    if (upw < stage_kb) return (int)hipErrorInvalidValue;
    const auto* b = static_cast<const fa::u32x4*>(buf);
    const hipStream_t st = (hipStream_t)stream;
    if (stage_kb == 4) return (int)fa::launch_read_lds_l<4>(b, upw, workgroups, stages, nontemporal, st);
    if (stage_kb == 8) return (int)fa::launch_read_lds_l<8>(b, upw, workgroups, stages, nontemporal, st);
    return (int)fa::launch_read_lds_l<16>(b, upw, workgroups, stages, nontemporal, st);
}

int fa_ceil_lds_read(void* sink, unsigned long long* stamps, int mode, int workgroups, int iters, void* stream) {
    if (!sink || !stamps || mode < 0 || mode > 3 || workgroups < 1 || iters < 1)
        return (int)hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fa::ceil_lds_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, fa::kLdsBytes);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(fa::ceil_lds_kernel, dim3(workgroups), dim3(256), fa::kLdsBytes, (hipStream_t)stream,
                       static_cast<uint32_t*>(sink), stamps, mode, iters);
    return (int)hipGetLastError();
}

}  // extern "C"
