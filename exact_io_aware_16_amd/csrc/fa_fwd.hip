// Forward pass of exact attention on gfx950.
//
// Method (handsonai.io "DL101 chapter 9", section 3.3 FlashAttention; the
// online softmax of the holysheep.ai Flash Attention article, section 2.1):
// for a block of query rows keep a running row max m, a running denominator l
// and an unnormalised output; for each arriving K/V block compute the scores,
// raise m, rescale l and the output by exp(m_old - m_new), add the block's
// exp(scores - m) and its product with V; divide by l once at the end.  The
// N x N score matrix only ever exists one register tile at a time.
//
// MI355X mapping (bf16 kernel):
//  * one workgroup = 4 waves = 128 query rows of one (batch, head); each wave
//    owns 32 query rows for the whole pass;
//  * K/V blocks of 64 keys are staged through LDS, double buffered, with the
//    next block's global loads in flight while the current block is computed;
//  * scores are computed transposed, S^T = K Q^T (32x32x16 bf16 MFMA, fp32
//    accumulate), so every lane owns one query column: the row max and row sum
//    are per-lane reductions plus one exchange with lane l^32;
//  * the output is accumulated transposed too, O^T += V^T P^T, so the rescale
//    by exp(m_old - m_new) is a per-lane scalar; V is written to LDS already
//    transposed (and key-permuted so each lane's eight keys are contiguous);
//  * the softmax runs in base 2 with scale*log2(e) folded into one FMA;
//  * causal: key blocks past the workgroup's last visible key are never
//    loaded, blocks past a wave's last visible key are skipped by that wave,
//    and only blocks crossing the diagonal pay for the mask;
//  * workgroups are issued heaviest query block first, and the blocks of one
//    (batch, head) are a multiple of 8 launch slots apart, so they land on the
//    same XCD and share its L2 copy of K and V.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D>
struct FwdTile {
    static constexpr int NW = 4;             // waves per workgroup
    static constexpr int BM = 32 * NW;       // query rows per workgroup
    static constexpr int BN = 64;            // keys per K/V block
    static constexpr int KS = D + 8;         // K tile row stride (elements), breaks bank aliasing
    static constexpr int VS = BN + 8;        // V^T tile row stride (elements)
    static constexpr int K_ELEMS = BN * KS;
    static constexpr int V_ELEMS = D * VS;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
    static constexpr int LDS_BYTES = 2 * STAGE * 2;
    static constexpr int KCH = BN * D / 8;   // 16-byte chunks in a K block
    static constexpr int KPT = KCH / 256;    // chunks per thread
    static constexpr int VIT = (BN / 4) * (D / 8);  // (4-key group, 8-column chunk) items
};

// Position of key kappa (0..63, a multiple of 4) inside a transposed V row:
// kappa = 32*mt + 8*g + 4*hh + r  ->  32*mt + 16*(g/2) + 8*hh + 4*(g%2) + r.
// Lane half hh then finds the eight keys it multiplies, in the order its P
// registers hold them, at one contiguous 16-byte slot.
__device__ __forceinline__ int vt_pos(int kappa) {
    const int mt = kappa >> 5, g = (kappa >> 3) & 3, hh = (kappa >> 2) & 1;
    return mt * 32 + (g >> 1) * 16 + hh * 8 + (g & 1) * 4;
}

template <int D>
struct KVStage {
    u32x4 k[FwdTile<D>::KPT];
    u32x4 v[4];
};

template <int D>
__device__ __forceinline__ void load_kv_block(KVStage<D>& st, const uint16_t* __restrict__ kb,
                                              const uint16_t* __restrict__ vb, int key0, int kv_end,
                                              int tid) {
    // Rows at or past kv_end are read from row kv_end - 1 instead: always in
    // bounds and finite; their scores are masked to -inf, so they enter the
    // result with probability exactly 0.
    using T = FwdTile<D>;
#pragma unroll
    for (int r = 0; r < T::KPT; ++r) {
        const int c = tid + 256 * r;
        const int row = c / (D / 8), col8 = c % (D / 8);
        const int key = min(key0 + row, kv_end - 1);
        st.k[r] = *reinterpret_cast<const u32x4*>(kb + (size_t)key * D + col8 * 8);
    }
    if (tid < T::VIT) {
        const int kq = tid / (D / 8), c8 = tid % (D / 8);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = min(key0 + kq * 4 + r, kv_end - 1);
            st.v[r] = *reinterpret_cast<const u32x4*>(vb + (size_t)key * D + c8 * 8);
        }
    }
}

template <int D>
__device__ __forceinline__ void store_kv_block(const KVStage<D>& st, uint16_t* sK, uint16_t* sV, int tid) {
    using T = FwdTile<D>;
#pragma unroll
    for (int r = 0; r < T::KPT; ++r) {
        const int c = tid + 256 * r;
        const int row = c / (D / 8), col8 = c % (D / 8);
        *reinterpret_cast<u32x4*>(sK + row * T::KS + col8 * 8) = st.k[r];
    }
    if (tid < T::VIT) {
        const int kq = tid / (D / 8), c8 = tid % (D / 8);
        const int pos = vt_pos(kq * 4);
        static_for<0, 8>([&](auto ec) {
            constexpr int e = decltype(ec)::value;
            const uint32_t lo = pack_col<e>(st.v[0], st.v[1]);
            const uint32_t hi = pack_col<e>(st.v[2], st.v[3]);
            *reinterpret_cast<u32x2*>(sV + (c8 * 8 + e) * T::VS + pos) = u32x2{lo, hi};
        });
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk, int nqb, int BH,
    float sl2) {
    using T = FwdTile<D>;
    extern __shared__ __align__(16) uint16_t smem[];

    const int id = blockIdx.x;
    const int qb = CAUSAL ? (nqb - 1 - id / BH) : (id / BH);
    const int bh = id % BH;
    const int b = bh / Hq, h = bh % Hq;
    const int hk = h / (Hq / Hkv);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int n = lane & 31, hf = lane >> 5;

    const uint16_t* qbase = Q + (size_t)(b * Hq + h) * Nq * D;
    const uint16_t* kbase = K + (size_t)(b * Hkv + hk) * Nk * D;
    const uint16_t* vbase = V + (size_t)(b * Hkv + hk) * Nk * D;

    const int off = Nk - Nq;  // bottom-right causal alignment
    const int qw = qb * T::BM + wave * 32;
    const int qi = qw + n;

    // Q^T as the B operand: lane (n, hf) holds q[qi][16*kk + 8*hf .. +7].
    bf16x8 qf[D / 16];
    {
        // rows past Nq read row Nq - 1; they are computed but never stored
        const uint16_t* qrow = qbase + (size_t)min(qi, Nq - 1) * D;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + kk * 16 + hf * 8));
    }

    int kv_end = Nk;
    if (CAUSAL) kv_end = min(Nk, qb * T::BM + T::BM + off);
    const int nblk = (kv_end + T::BN - 1) / T::BN;
    int wave_end = Nk;  // one past the last key any row of this wave sees
    if (CAUSAL) wave_end = min(Nk, qw + 32 + off);
    const int mask_from = CAUSAL ? (qw + off) : Nk;  // first key some row of the wave cannot see

    f32x16 ot[D / 32];
#pragma unroll
    for (int md = 0; md < D / 32; ++md) ot[md] = zero16();
    float m_run = kNegInf;  // running max of scale*log2(e)*s for query qi
    float l_run = 0.f;      // running sum over this lane's half of the keys

    KVStage<D> st;
    load_kv_block<D>(st, kbase, vbase, 0, kv_end, tid);
    store_kv_block<D>(st, smem, smem + T::K_ELEMS, tid);
    __syncthreads();

    for (int j = 0; j < nblk; ++j) {
        const int key0 = j * T::BN;
        uint16_t* sK = smem + (j & 1) * T::STAGE;
        uint16_t* sV = sK + T::K_ELEMS;
        if (j + 1 < nblk) load_kv_block<D>(st, kbase, vbase, key0 + T::BN, kv_end, tid);

        if (key0 < wave_end) {
            // ---- S^T = K Q^T for 64 keys x 32 queries --------------------------------
            f32x16 s[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                s[mt] = zero16();
                const uint16_t* ka = sK + (mt * 32 + n) * T::KS + hf * 8;
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(ka + kk * 16);
                    s[mt] = mfma32x32x16(a, qf[kk], s[mt]);
                }
            }
            // ---- mask (only on blocks that cross the diagonal or the end) ----------
            if (key0 + T::BN > mask_from || key0 + T::BN > kv_end) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = key0 + mt * 32 + (i >> 2) * 8 + hf * 4 + (i & 3);
                        const bool ok = key < kv_end && (!CAUSAL || key <= qi + off);
                        s[mt][i] = ok ? s[mt][i] : kNegInf;
                    }
            }
            // ---- online softmax (base 2) -------------------------------------------
            float mx = kNegInf;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; i += 2) mx = max3f(mx, s[mt][i], s[mt][i + 1]);
            mx = __builtin_fmaxf(mx, xor32(mx));
            const float m_new = __builtin_fmaxf(m_run, mx * sl2);
            const float m_use = (m_new == kNegInf) ? 0.f : m_new;
            if (!wave_all(m_new == m_run)) {
                const float corr = exp2_fast(m_run - m_use);
                l_run *= corr;
#pragma unroll
                for (int md = 0; md < D / 32; ++md)
#pragma unroll
                    for (int i = 0; i < 16; ++i) ot[md][i] *= corr;
            }
            m_run = m_new;
            float psum = 0.f;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = exp2_fast(__builtin_fmaf(s[mt][i], sl2, -m_use));
                    s[mt][i] = p;
                    psum += p;
                }
            l_run += psum;
            // ---- O^T += V^T P^T ----------------------------------------------------
#pragma unroll
            for (int ks = 0; ks < T::BN / 16; ++ks) {
                const int mt = ks >> 1, base = (ks & 1) * 8;
                bf16x8 pb;
#pragma unroll
                for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[mt][base + e];
                const uint16_t* va = sV + n * T::VS + ks * 16 + hf * 8;
#pragma unroll
                for (int md = 0; md < D / 32; ++md) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(va + md * 32 * T::VS);
                    ot[md] = mfma32x32x16(a, pb, ot[md]);
                }
            }
        }

        if (j + 1 < nblk) {
            uint16_t* nK = smem + ((j + 1) & 1) * T::STAGE;
            store_kv_block<D>(st, nK, nK + T::K_ELEMS, tid);
        }
        __syncthreads();
    }

    // ---- finalise: O = O / l, LSE = (m + log2 l) * ln 2 ---------------------------
    const float l_tot = l_run + xor32(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qi < Nq) {
        uint16_t* orow = O + ((size_t)(b * Hq + h) * Nq + qi) * D;
#pragma unroll
        for (int md = 0; md < D / 32; ++md)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dcol = md * 32 + g * 8 + hf * 4;
                const uint32_t lo = pack_bf16x2(ot[md][g * 4 + 0] * inv, ot[md][g * 4 + 1] * inv);
                const uint32_t hi = pack_bf16x2(ot[md][g * 4 + 2] * inv, ot[md][g * 4 + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + dcol) = u32x2{lo, hi};
            }
        if (hf == 0)
            LSE[(size_t)(b * Hq + h) * Nq + qi] = l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : kNegInf;
    }
}

// ---------------------------------------------------------------------------
// float32 forward: the same recurrence on the vector ALUs, four lanes per query
// row (each owns d/4 columns).  Also serves float32 decode through kv_lens.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ V, float* __restrict__ O,
                                                      float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk,
                                                      int causal, float sl2, const int* __restrict__ kv_lens) {
    constexpr int DS = D / 4;   // columns per lane
    constexpr int BK = 32;      // keys per LDS block
    __shared__ float sK[BK][D + 4];
    __shared__ float sV[BK][D + 4];

    const int b = blockIdx.z, h = blockIdx.y;
    const int hk = h / (Hq / Hkv);
    const int tid = threadIdx.x;
    const int row = tid >> 2, part = tid & 3;
    const int qi = blockIdx.x * 64 + row;
    const int off = Nk - Nq;

    int kv_end = Nk;
    if (kv_lens) kv_end = max(0, min(Nk, kv_lens[b]));
    int wg_end = kv_end;
    if (causal) wg_end = min(kv_end, blockIdx.x * 64 + 64 + off);

    const float* qrow = Q + ((size_t)(b * Hq + h) * Nq + (qi < Nq ? qi : 0)) * D + part * DS;
    const float* kb = K + (size_t)(b * Hkv + hk) * Nk * D;
    const float* vb = V + (size_t)(b * Hkv + hk) * Nk * D;

    float q[DS], o[DS];
#pragma unroll
    for (int c = 0; c < DS; ++c) {
        q[c] = qrow[c];
        o[c] = 0.f;
    }
    float m_run = kNegInf, l_run = 0.f;

    for (int key0 = 0; key0 < wg_end; key0 += BK) {
        __syncthreads();
        for (int e = tid; e < BK * D; e += 256) {
            const int r = e / D, c = e % D;
            const int key = key0 + r;
            sK[r][c] = key < kv_end ? kb[(size_t)key * D + c] : 0.f;
            sV[r][c] = key < kv_end ? vb[(size_t)key * D + c] : 0.f;
        }
        __syncthreads();
        float s[BK];
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < BK; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < DS; ++c) acc = __builtin_fmaf(q[c], sK[j][part * DS + c], acc);
            acc += __shfl_xor(acc, 1, 64);
            acc += __shfl_xor(acc, 2, 64);
            const int key = key0 + j;
            const bool ok = key < kv_end && (!causal || key <= qi + off);
            s[j] = ok ? acc : kNegInf;
            mx = __builtin_fmaxf(mx, s[j]);
        }
        const float m_new = __builtin_fmaxf(m_run, mx * sl2);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float corr = exp2_fast(m_run - m_use);
        l_run *= corr;
#pragma unroll
        for (int c = 0; c < DS; ++c) o[c] *= corr;
        m_run = m_new;
#pragma unroll
        for (int j = 0; j < BK; ++j) {
            const float p = exp2_fast(__builtin_fmaf(s[j], sl2, -m_use));
            l_run += p;
#pragma unroll
            for (int c = 0; c < DS; ++c) o[c] = __builtin_fmaf(p, sV[j][part * DS + c], o[c]);
        }
    }
    if (qi < Nq) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        float* orow = O + ((size_t)(b * Hq + h) * Nq + qi) * D + part * DS;
#pragma unroll
        for (int c = 0; c < DS; ++c) orow[c] = o[c] * inv;
        if (part == 0)
            LSE[(size_t)(b * Hq + h) * Nq + qi] = l_run > 0.f ? (m_run + log2_fast(l_run)) * kLn2 : kNegInf;
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
static hipError_t launch_fwd_bf16_t(const FwdArgs& a) {
    using T = FwdTile<D>;
    const int nqb = (a.Nq + T::BM - 1) / T::BM;
    const int BH = a.B * a.Hq;
    auto kern = fwd_bf16_kernel<D, CAUSAL>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, T::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(nqb * BH), dim3(256), T::LDS_BYTES, (hipStream_t)a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse,
                       a.Hq, a.Hkv, a.Nq, a.Nk, nqb, BH, a.scale * kLog2e);
    return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a) {
    if (a.d == 64) return a.causal ? launch_fwd_bf16_t<64, true>(a) : launch_fwd_bf16_t<64, false>(a);
    return a.causal ? launch_fwd_bf16_t<128, true>(a) : launch_fwd_bf16_t<128, false>(a);
}

template <int D>
static hipError_t launch_fwd_f32_t(const FwdArgs& a, const int* kv_lens) {
    dim3 grid((a.Nq + 63) / 64, a.Hq, a.B);
    hipLaunchKernelGGL(fwd_f32_kernel<D>, grid, dim3(256), 0, (hipStream_t)a.stream, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.Hq, a.Hkv, a.Nq, a.Nk,
                       a.causal, a.scale * kLog2e, kv_lens);
    return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdArgs& a, const int* kv_lens) {
    return a.d == 64 ? launch_fwd_f32_t<64>(a, kv_lens) : launch_fwd_f32_t<128>(a, kv_lens);
}

}  // namespace fa
