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

#include <algorithm>

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

// All V^T fragments of one 32-key stage (frag_tr_swz for k0 = 0, 16 and every
// 32-column block), read with ds_read_b64_tr_b16 in a single asm block that
// ends in its own lgkmcnt(0).  Written as asm because the compiler guards
// every transpose-read builtin that follows a direct-to-LDS load with a full
// vmcnt(0), which would drain the look-ahead ring each stage; here the ring's
// explicit vmcnt wait already orders the reads after the stage's loads.
template <int D>
__device__ __forceinline__ void stage_vt_frags(const uint16_t* X, int lane, bf16x8 (&vf)[2][D / 32]) {
    constexpr int NF = 2 * (D / 32);              // fragments, two reads each
    const int t = lane & 15;
    unsigned ad[2 * NF];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int md = 0; md < D / 32; ++md) {
            const int row = ks * 16 + (lane >> 5) * 4 + (t >> 2);
            const int col = md * 32 + ((lane >> 4) & 1) * 16 + (t & 3) * 4;
            const int f = ks * (D / 32) + md;
            ad[2 * f] = (unsigned)(uintptr_t)(X + swz_off<D>(row, col >> 3) + (col & 7));
            ad[2 * f + 1] = (unsigned)(uintptr_t)(X + swz_off<D>(row + 8, col >> 3) + (col & 7));
        }
    u32x2 r[2 * NF];
    if constexpr (D == 128) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %16\n\tds_read_b64_tr_b16 %1, %17\n\t"
            "ds_read_b64_tr_b16 %2, %18\n\tds_read_b64_tr_b16 %3, %19\n\t"
            "ds_read_b64_tr_b16 %4, %20\n\tds_read_b64_tr_b16 %5, %21\n\t"
            "ds_read_b64_tr_b16 %6, %22\n\tds_read_b64_tr_b16 %7, %23\n\t"
            "ds_read_b64_tr_b16 %8, %24\n\tds_read_b64_tr_b16 %9, %25\n\t"
            "ds_read_b64_tr_b16 %10, %26\n\tds_read_b64_tr_b16 %11, %27\n\t"
            "ds_read_b64_tr_b16 %12, %28\n\tds_read_b64_tr_b16 %13, %29\n\t"
            "ds_read_b64_tr_b16 %14, %30\n\tds_read_b64_tr_b16 %15, %31\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
              "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]),
              "=&v"(r[14]), "=&v"(r[15])
            : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7]),
              "v"(ad[8]), "v"(ad[9]), "v"(ad[10]), "v"(ad[11]), "v"(ad[12]), "v"(ad[13]), "v"(ad[14]), "v"(ad[15])
            : "memory");
    } else {
        static_assert(D == 64, "head dimension");
        asm volatile(
            "ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %9\n\t"
            "ds_read_b64_tr_b16 %2, %10\n\tds_read_b64_tr_b16 %3, %11\n\t"
            "ds_read_b64_tr_b16 %4, %12\n\tds_read_b64_tr_b16 %5, %13\n\t"
            "ds_read_b64_tr_b16 %6, %14\n\tds_read_b64_tr_b16 %7, %15\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
              "=&v"(r[7])
            : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7])
            : "memory");
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const u32x4 w = {r[2 * f][0], r[2 * f][1], r[2 * f + 1][0], r[2 * f + 1][1]};
        vf[f / (D / 32)][f % (D / 32)] = __builtin_bit_cast(bf16x8, w);
    }
}

// ---------------------------------------------------------------------------
// Streaming split kernel.  A workgroup is one wave and owns one split
// (keys [512 c, 512 c + 512) of one K/V head of one sequence, for up to 32
// query heads of its group).  The split is streamed in 32-key stages through
// a private ring of DS stages in LDS, filled by direct-to-LDS loads
// (global_load_lds_dwordx4) DS-1 stages ahead of the matrix cores; the wave
// only reads what it loaded itself, so no barriers are needed, and the loop
// issues no register-destination loads, so every wait is an explicit vmcnt.
// Several such waves share a CU and the hardware dispatcher hands out splits
// as waves finish, which balances ragged sequence lengths.  K and V stages are
// dense and XOR-swizzled (conflict-free row and transpose reads).
// ---------------------------------------------------------------------------
template <int D, int DS, int QR>
struct RingDecTile {
    static constexpr int BK = 32;                    // keys per stage
    static constexpr int TILE = BK * D;              // elements of K (or V) per stage
    static constexpr int STAGE = 2 * TILE;
    static constexpr int QTILE = QR * D;             // the group's query rows, loaded once
    static constexpr int LDS_BYTES = (DS * STAGE + QTILE) * 2;
    static constexpr int IPT = BK * D / 8 / 64;      // load instructions per K (or V) tile
    static constexpr int QI = QR * D / 8 / 64;       // load instructions for the query rows
    static constexpr int LPS = 2 * IPT;              // per stage
    static_assert(QI >= 1 && QR * D / 8 == QI * 64, "query rows must fill whole loads");
    static_assert((DS - 1) * LPS < 64, "vmcnt range");
};

#define DEC_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// wait until at most r stages (r < DS-1, runtime) are still in flight
template <int LPS, int DS>
__device__ __forceinline__ void wait_stages(int r) {
    if constexpr (DS >= 5) if (r >= 3) { wait_vmcnt<3 * LPS>(); return; }
    if constexpr (DS >= 4) if (r >= 2) { wait_vmcnt<2 * LPS>(); return; }
    if constexpr (DS >= 3) if (r >= 1) { wait_vmcnt<1 * LPS>(); return; }
    wait_vmcnt<0>();
}

template <int D, int DS, int QR>
__global__ __launch_bounds__(64) void decode_ring_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const int* __restrict__ seqlens, float* __restrict__ part_o, float* __restrict__ part_lse, int Hq, int Hkv,
    int Nmax, int nsplit, int nht, float sl2) {
    using T = RingDecTile<D, DS, QR>;
    static_assert(DS <= 5, "wait_stages covers at most five stages");
    extern __shared__ __align__(16) uint16_t smem[];
    const int c = blockIdx.x;
    const int hk = blockIdx.y / nht, ht = blockIdx.y % nht;
    const int b = blockIdx.z;
    const int g = Hq / Hkv;
    const int len = max(0, min(Nmax, seqlens[b]));
    const int k_begin = c * kDecodeSplit;
    if (k_begin >= len) return;
    const int k_end = min(len, k_begin + kDecodeSplit);
    const int nst = (k_end - k_begin + T::BK - 1) / T::BK;

    const int lane = threadIdx.x;
    const int n = lane & 31, hf = lane >> 5;
    const int gh = ht * 32 + n;
    const bool head_ok = gh < g;
    uint16_t* sQ = smem + DS * T::STAGE;

    // the group's query rows ht*32 .. ht*32+QR-1 (rows past the group read its
    // last head; they only feed output columns that are never stored)
#pragma unroll
    for (int i = 0; i < T::QI; ++i) {
        const int slot = i * 64 + lane;
        const int row = slot / (D / 8), pos = slot % (D / 8);
        const int head = min(ht * 32 + row, g - 1);
        const size_t gi = (size_t)(b * Hq + hk * g + head) * D + ((pos ^ swz<D>(row)) << 3);
        __builtin_amdgcn_global_load_lds(Q + gi, DEC_LDS_PTR(sQ + i * 64 * 8), 16, 0, 0);
    }

    const uint16_t* kbase = K + (size_t)(b * Hkv + hk) * Nmax * D;
    const uint16_t* vbase = V + (size_t)(b * Hkv + hk) * Nmax * D;
    // stage j -> ring slot j % DS; keys at or past k_end are read from row
    // k_end - 1 (their scores are masked to -inf, so they weigh exactly 0)
    auto issue = [&](int j) {
        uint16_t* kt = smem + (j % DS) * T::STAGE;
        uint16_t* vt = kt + T::TILE;
        const int key0 = k_begin + j * T::BK;
#pragma unroll
        for (int i = 0; i < T::IPT; ++i) {
            const int slot = i * 64 + lane;
            const int row = slot / (D / 8), pos = slot % (D / 8);
            const size_t gi = (size_t)min(key0 + row, k_end - 1) * D + ((pos ^ swz<D>(row)) << 3);
            __builtin_amdgcn_global_load_lds(kbase + gi, DEC_LDS_PTR(kt + i * 64 * 8), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(vbase + gi, DEC_LDS_PTR(vt + i * 64 * 8), 16, 0, 0);
        }
    };
    const int pro = min(DS - 1, nst);
    for (int j = 0; j < pro; ++j) issue(j);

    // query operand Q^T: lane (n, hf) takes query row min(n, QR-1); the query
    // loads are the oldest, so waiting down to the prologue's stages suffices
    wait_stages<T::LPS, DS + 1>(pro);
    bf16x8 qf[D / 16];
    {
        const int qr = min(n, QR - 1);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qf[kk] = *reinterpret_cast<const bf16x8*>(sQ + swz_off<D>(qr, kk * 2 + hf));
    }

    f32x16 ot[D / 32];
#pragma unroll
    for (int md = 0; md < D / 32; ++md) ot[md] = zero16();
    float m_run = kNegInf, l_run = 0.f;

    for (int j = 0; j < nst; ++j) {
        // stage j has landed once at most min(DS-2, nst-1-j) younger stages remain
        wait_stages<T::LPS, DS>(min(DS - 2, nst - 1 - j));
        __builtin_amdgcn_sched_barrier(0);
        if (j + DS - 1 < nst) issue(j + DS - 1);
        const uint16_t* sK = smem + (j % DS) * T::STAGE;
        const uint16_t* sV = sK + T::TILE;
        const int key0 = k_begin + j * T::BK;
        bf16x8 kf[D / 16];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) kf[kk] = frag_rows_swz<D>(sK, 0, kk * 16, lane);
        f32x16 sc = zero16();
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) sc = mfma32x32x16(kf[kk], qf[kk], sc);
        if (key0 + T::BK > k_end) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = key0 + (i >> 2) * 8 + hf * 4 + (i & 3);
                sc[i] = key < k_end ? sc[i] : kNegInf;
            }
        }
        float m0 = kNegInf, m1 = kNegInf;
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
            m0 = max3f(m0, sc[i], sc[i + 1]);
            m1 = max3f(m1, sc[i + 2], sc[i + 3]);
        }
        const float mx = pair_max(__builtin_fmaxf(m0, m1)) * sl2;
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
        bf16x8 vf[2][D / 32];
        stage_vt_frags<D>(sV, lane, vf);
        bf16x8 pb[2];
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            const float p0 = exp2_fast(__builtin_fmaf(sc[i], sl2, -m_use));
            const float p1 = exp2_fast(__builtin_fmaf(sc[i + 1], sl2, -m_use));
            ps0 += p0;
            ps1 += p1;
            pb[i >> 3][i & 7] = (__bf16)p0;
            pb[i >> 3][(i & 7) + 1] = (__bf16)p1;
        }
        l_run += ps0 + ps1;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int md = 0; md < D / 32; ++md) ot[md] = mfma32x32x16(vf[ks][md], pb[ks], ot[md]);
    }

    // the split's partial: O_s = O / l, lse_s = m + log l
    const float l_tot = pair_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (head_ok) {
        const size_t row = (size_t)(b * Hq + hk * g + gh) * nsplit + c;
        float* po = part_o + row * D;
#pragma unroll
        for (int md = 0; md < D / 32; ++md)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *reinterpret_cast<f32x4*>(po + md * 32 + q4 * 8 + hf * 4) =
                    f32x4{ot[md][q4 * 4] * inv, ot[md][q4 * 4 + 1] * inv, ot[md][q4 * 4 + 2] * inv,
                          ot[md][q4 * 4 + 3] * inv};
        if (hf == 0) part_lse[row] = l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : kNegInf;
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

#ifndef DEC_RING
#define DEC_RING 1
#endif
#ifndef DEC_STAGES
#define DEC_STAGES 3
#endif

template <int D, int QR>
static hipError_t launch_decode_ring(const DecodeArgs& a, int nht) {
    using T = RingDecTile<D, DEC_STAGES, QR>;
    auto kern = decode_ring_kernel<D, DEC_STAGES, QR>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, T::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.nsplit, a.Hkv * nht, a.B), dim3(64), T::LDS_BYTES, (hipStream_t)a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.seqlens, a.part_o,
                       a.part_lse, a.Hq, a.Hkv, a.Nmax, a.nsplit, nht, a.scale * kLog2e);
    return hipSuccess;
}

template <int D>
static hipError_t launch_decode_t(const DecodeArgs& a) {
    const int g = a.Hq / a.Hkv;
    const int nht = (g + 31) / 32;
    hipError_t e;
#if DEC_RING
    {
        // query rows staged in LDS: the group size rounded up to whole loads, at most 32
        constexpr int RPL = 64 * 8 / D;   // rows per load instruction
        const int rows = std::min(g, 32);
        if (rows <= RPL) e = launch_decode_ring<D, RPL>(a, nht);
        else if (rows <= 2 * RPL) e = launch_decode_ring<D, std::min(2 * RPL, 32)>(a, nht);
        else if (rows <= 4 * RPL) e = launch_decode_ring<D, std::min(4 * RPL, 32)>(a, nht);
        else e = launch_decode_ring<D, 32>(a, nht);
        if (e != hipSuccess) return e;
    }
#else
    {
        using T = DecTile<D>;
        auto kern = decode_split_kernel<D>;
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                T::LDS_BYTES);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(a.nsplit, a.Hkv * nht, a.B), dim3(256), T::LDS_BYTES, (hipStream_t)a.stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.seqlens, a.part_o,
                           a.part_lse, a.Hq, a.Hkv, a.Nmax, a.nsplit, nht, a.scale * kLog2e);
    }
#endif
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
