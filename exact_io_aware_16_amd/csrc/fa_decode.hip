// Decode: one new query token per head against a long KV cache (handsonai.io
// "DL101 chapter 9", section 1.1 Key/Value Caching: the token at step t
// attends to every cached key/value up to t), with grouped K/V heads (same
// page, sections 3.1 MQA and 3.2 GQA).
//
// The work is bound by reading the cache once.  MI355X mapping:
//  * split-K over the cache: workgroup (split s, K/V head, batch) streams keys
//    [512 s, 512 s + 512) of one K/V head exactly once, for all query heads of
//    its group at the same time (up to 32 heads in one matrix-core column
//    tile), so the grouped heads cost no extra cache traffic;
//  * 128-key sub-blocks are loaded with fully coalesced 16-byte loads into
//    registers one sub-block ahead, then staged through LDS (K as is, V
//    transposed) for the 32x32x16 bf16 matrix cores; each wave owns 32 keys;
//  * splits past a sequence's length exit at once; keys at or past the length
//    are never read into the result (their V rows are replaced by zeros and
//    their scores by -inf), so any contents there, NaN included, are harmless;
//  * each split ends with the four waves' (max, sum, output) merged in LDS and
//    one partial (O_s, lse_s) written; a second kernel merges the splits with
//    weights exp(lse_s - lse), the same rescaling the online softmax applies
//    when a new block arrives (holysheep.ai Flash Attention article, section
//    2.1 Online Softmax).
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int DBN = 128;  // keys per sub-block (4 waves x 32)

template <int D>
struct DecTile {
    static constexpr int KS = D + 8;    // K row stride (row reads: distinct bank quads)
    static constexpr int VS = D + 32;   // V row stride (64 B mod 256 B: transpose reads 2-way)
    static constexpr int K_ELEMS = DBN * KS;
    static constexpr int V_ELEMS = DBN * VS;
    static constexpr int LDS_BYTES = (K_ELEMS + V_ELEMS) * 2;
    static constexpr int CPT = DBN * D / 8 / 256;   // 16-byte chunks per thread per tensor
};

constexpr float kRescaleThreshold = 8.0f;   // lazy rescaling, as in the forward kernel

}  // namespace

template <int D>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const int* __restrict__ seqlens, float* __restrict__ part_o, float* __restrict__ part_lse, int Hq, int Hkv,
    int Nmax, int nsplit, int nht, float sl2) {
    using T = DecTile<D>;
    extern __shared__ __align__(16) uint16_t smem[];
    uint16_t* sK = smem;
    uint16_t* sV = smem + T::K_ELEMS;

    const int s = blockIdx.x;
    const int hk = blockIdx.y / nht, ht = blockIdx.y % nht;
    const int b = blockIdx.z;
    const int g = Hq / Hkv;
    const int len = max(0, min(Nmax, seqlens[b]));
    const int k_begin = s * kDecodeSplit;
    if (k_begin >= len) return;
    const int k_end = min(len, k_begin + kDecodeSplit);
    const int nsub = (k_end - k_begin + DBN - 1) / DBN;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 31, hf = lane >> 5;
    const int gh = ht * 32 + n;          // head index inside the group
    const int hq = hk * g + gh;
    const bool head_ok = gh < g;

    bf16x8 qf[D / 16];
    {
        // lanes past the group's last head read that head's row; never stored
        const uint16_t* qrow = Q + (size_t)(b * Hq + (head_ok ? hq : hk * g + g - 1)) * D;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + kk * 16 + hf * 8));
    }

    const uint16_t* kb = K + (size_t)(b * Hkv + hk) * Nmax * D;
    const uint16_t* vb = V + (size_t)(b * Hkv + hk) * Nmax * D;

    // Keys at or past k_end are read from row k_end - 1 (a valid, finite row of
    // this sequence): their scores are masked to -inf so they carry weight
    // exactly 0, and the cache beyond the sequence length is never touched.
    // 16 consecutive threads move one 256-byte key row (full-row loads, one
    // contiguous LDS run per row).
    u32x4 kr[T::CPT], vr[T::CPT];
    auto load = [&](int key0) {
#pragma unroll
        for (int r = 0; r < T::CPT; ++r) {
            const int c = tid + 256 * r;
            const int row = c / (D / 8), col8 = c % (D / 8);
            const size_t gi = (size_t)min(key0 + row, k_end - 1) * D + col8 * 8;
            kr[r] = *reinterpret_cast<const u32x4*>(kb + gi);
            vr[r] = *reinterpret_cast<const u32x4*>(vb + gi);
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int r = 0; r < T::CPT; ++r) {
            const int c = tid + 256 * r;
            const int row = c / (D / 8), col8 = c % (D / 8);
            *reinterpret_cast<u32x4*>(sK + row * T::KS + col8 * 8) = kr[r];
            *reinterpret_cast<u32x4*>(sV + row * T::VS + col8 * 8) = vr[r];
        }
    };

    f32x16 ot[D / 32];
#pragma unroll
    for (int md = 0; md < D / 32; ++md) ot[md] = zero16();
    float m_run = kNegInf, l_run = 0.f;

    load(k_begin);
    for (int it = 0; it < nsub; ++it) {
        const int key0 = k_begin + it * DBN;
        store();
        __syncthreads();
        if (it + 1 < nsub) load(key0 + DBN);
        const int wkey0 = key0 + wave * 32;
        if (wkey0 < k_end) {
            f32x16 sc = zero16();
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                sc = mfma32x32x16(frag_rows(sK, T::KS, wave * 32, kk * 16, lane), qf[kk], sc);
            if (wkey0 + 32 > k_end) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = wkey0 + (i >> 2) * 8 + hf * 4 + (i & 3);
                    sc[i] = key < k_end ? sc[i] : kNegInf;
                }
            }
            float mx = kNegInf;
#pragma unroll
            for (int i = 0; i < 16; i += 2) mx = max3f(mx, sc[i], sc[i + 1]);
            mx = pair_max(mx) * sl2;
            if (!wave_all(mx <= m_run + kRescaleThreshold)) {
                const float m_new = __builtin_fmaxf(m_run, mx);
                const float corr = (m_new == kNegInf) ? 1.f : exp2_fast(m_run - m_new);
                l_run *= corr;
#pragma unroll
                for (int md = 0; md < D / 32; ++md)
#pragma unroll
                    for (int i = 0; i < 16; ++i) ot[md][i] *= corr;
                m_run = m_new;
            }
            const float m_use = (m_run == kNegInf) ? 0.f : m_run;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = exp2_fast(__builtin_fmaf(sc[i], sl2, -m_use));
                sc[i] = p;
                l_run += p;
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 pb;
#pragma unroll
                for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sc[ks * 8 + e];
#pragma unroll
                for (int md = 0; md < D / 32; ++md)
                    ot[md] = mfma32x32x16(frag_tr(sV, T::VS, wave * 32 + ks * 16, md * 32, lane), pb, ot[md]);
            }
        }
        __syncthreads();
    }

    // ---- merge the four waves' partial softmax states in LDS ------------------
    float* sm = reinterpret_cast<float*>(smem);   // [4][32] max
    float* sl = sm + 128;                         // [4][32] sum
    float* so = sl + 128;                         // [4][32][D] scaled outputs
    const float l_tot = pair_sum(l_run);
    if (hf == 0) {
        sm[wave * 32 + n] = m_run;
        sl[wave * 32 + n] = l_tot;
    }
    __syncthreads();
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = __builtin_fmaxf(M, sm[w * 32 + n]);
    const float wscale = (m_run == kNegInf) ? 0.f : exp2_fast(m_run - M);
#pragma unroll
    for (int md = 0; md < D / 32; ++md)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int dcol = md * 32 + (i >> 2) * 8 + hf * 4 + (i & 3);
            so[(wave * 32 + n) * D + dcol] = ot[md][i] * wscale;
        }
    __syncthreads();
    for (int e = tid; e < 32 * D; e += 256) {
        const int hn = e / D, dcol = e % D;
        const int ghn = ht * 32 + hn;
        if (ghn >= g) continue;
        float Mn = kNegInf;
#pragma unroll
        for (int w = 0; w < 4; ++w) Mn = __builtin_fmaxf(Mn, sm[w * 32 + hn]);
        float L = 0.f, acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float mw = sm[w * 32 + hn];
            L += (mw == kNegInf) ? 0.f : sl[w * 32 + hn] * exp2_fast(mw - Mn);
            acc += so[(w * 32 + hn) * D + dcol];
        }
        const size_t row = (size_t)(b * Hq + hk * g + ghn) * nsplit + s;
        part_o[row * D + dcol] = acc / L;
        if (dcol == 0) part_lse[row] = (Mn + log2_fast(L)) * kLn2;
    }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_lse,
                                                           const int* __restrict__ seqlens, uint16_t* __restrict__ O,
                                                           float* __restrict__ LSE, int Hq, int Nmax, int nsplit) {
    const int hq = blockIdx.x, b = blockIdx.y;
    const int dcol = threadIdx.x;
    const int len = max(0, min(Nmax, seqlens[b]));
    const int ns = (len + kDecodeSplit - 1) / kDecodeSplit;
    const size_t row0 = (size_t)(b * Hq + hq) * nsplit;
    uint16_t* orow = O + (size_t)(b * Hq + hq) * D;
    if (ns == 0) {
        orow[dcol] = 0;
        if (dcol == 0) LSE[b * Hq + hq] = kNegInf;
        return;
    }
    float M = kNegInf;
    for (int s = 0; s < ns; ++s) M = __builtin_fmaxf(M, part_lse[row0 + s]);
    float L = 0.f, acc = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float w = exp2_fast((part_lse[row0 + s] - M) * kLog2e);
        L += w;
        acc = __builtin_fmaf(w, part_o[(row0 + s) * D + dcol], acc);
    }
    orow[dcol] = f32_to_bf16_bits(acc / L);
    if (dcol == 0) LSE[b * Hq + hq] = M + log2_fast(L) * kLn2;
}

template <int D>
static hipError_t launch_decode_t(const DecodeArgs& a) {
    using T = DecTile<D>;
    const int g = a.Hq / a.Hkv;
    const int nht = (g + 31) / 32;
    auto kern = decode_split_kernel<D>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, T::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.nsplit, a.Hkv * nht, a.B), dim3(256), T::LDS_BYTES, (hipStream_t)a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.seqlens, a.part_o,
                       a.part_lse, a.Hq, a.Hkv, a.Nmax, a.nsplit, nht, a.scale * kLog2e);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(a.Hq, a.B), dim3(D), 0, (hipStream_t)a.stream, a.part_o,
                       a.part_lse, a.seqlens, (uint16_t*)a.o, a.lse, a.Hq, a.Nmax, a.nsplit);
    return hipGetLastError();
}

hipError_t launch_decode_bf16(const DecodeArgs& a) {
    return a.d == 64 ? launch_decode_t<64>(a) : launch_decode_t<128>(a);
}

}  // namespace fa
