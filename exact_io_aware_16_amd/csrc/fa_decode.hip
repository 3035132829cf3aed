// Decode: one new query token per head against a long KV cache (handsonai.io
// "DL101 chapter 9", section 1.1 Key/Value Caching: the token at step t
// attends to every cached key/value up to t), with grouped K/V heads (same
// page, sections 3.1 MQA and 3.2 GQA).
//
// The work is bound by reading the cache once.  MI355X mapping:
//  * every cached key row is read exactly once, for all query heads of its
//    group at the same time (up to 32 heads in one matrix-core column tile),
//    so grouped heads cost no extra cache traffic;
//  * stream-K work split: the rows' keys are cut into 32-key stages laid end
//    to end and each one-wave workgroup takes an equal contiguous share, so
//    ragged sequence lengths leave no wave idle and no tail of short splits;
//  * each wave streams its share through a private ring of LDS stages filled
//    by direct-to-LDS loads (global_load_lds_dwordx4) ahead of the 32x32x16
//    bf16 matrix cores, with explicit vmcnt waits and no barriers;
//  * keys at or past a sequence's length are never read into the result (the
//    row is clamped to the last valid key and its score masked to -inf), so
//    any cache contents there, NaN included, are harmless;
//  * each wave writes one partial (O_s, lse_s) per row piece it covered; a
//    second kernel merges a row's pieces with weights exp(lse_s - lse), the
//    same rescaling the online softmax applies when a new block arrives
//    (holysheep.ai Flash Attention article, section 2.1 Online Softmax).
#include "fa_device.h"
#include "fa_launch.h"

#include <algorithm>

namespace fa {

namespace {
// cache-policy operand of global_load_lds for a non-temporal load on gfx950
constexpr int kLoadNonTemporal = 2;
constexpr float kRescaleThreshold = 8.0f;   // lazy rescaling: the max is raised on a jump past 2^8
}  // namespace

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

#define DEC_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// wait until at most r stages (r < DS-1, runtime) are still in flight
template <int LPS, int DS>
__device__ __forceinline__ void wait_stages(int r) {
    if constexpr (DS >= 5) if (r >= 3) { wait_vmcnt<3 * LPS>(); return; }
    if constexpr (DS >= 4) if (r >= 2) { wait_vmcnt<2 * LPS>(); return; }
    if constexpr (DS >= 3) if (r >= 1) { wait_vmcnt<1 * LPS>(); return; }
    wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// Stream-K variant.  The key range of every (sequence, K/V head, head tile)
// row is cut into 32-key stages and all stages of all rows are laid end to
// end; wave w of G takes a contiguous range of the S stages (dec_range_start:
// equal shares, or a set skew between the XCDs of a pair), so the waves stream
// the same number of bytes (or the set ratio) whatever the mix of
// sequence lengths, and its ring of DS stages runs across row boundaries
// without draining.  A stage holds 32 keys of K and V and the row's query
// rows (dense, XOR-swizzled), all brought in by direct-to-LDS loads DS-1
// stages ahead.  At the end of a row, or of its range, a wave writes the
// partial (O_s, lse_s) of the stages it saw to slot r + w (row r, wave w):
// the waves touching one row are consecutive, so these slots never collide
// and there are at most rows + G of them.  Wave 0 also writes the prefix sums
// of stages per sequence, from which the combine finds each row's waves.
// ---------------------------------------------------------------------------
// Share of the stages taken by the wave on the even XCD of each pair, in 64ths
// (measured on MI355X: waves on odd XCDs stream 10-12% slower; 35/64 was
// fastest, +2-3% over an even split).
constexpr int kDecEven64 = 35;

// Start of wave w's range of the S stages (w = G gives S).  Waves go in pairs
// (2p, 2p+1), which the dispatcher places on an even and an odd XCD (one-wave
// workgroup w runs on XCD w mod 8); pair p covers [p S / (G/2), (p+1) S / (G/2))
// and its even wave the first kDecEven64/64 of that.  G is even.
// (The same integer arithmetic in 32 bits whenever S * (G/2) < 2^31, the usual
// case: 64-bit divisions are emulated and cost the combine kernel, which
// evaluates these per piece, far more.)
__device__ __forceinline__ long long dec_range_start(int w, long long S, int G) {
    const int gp = G >> 1, p = w >> 1;
    if (S * gp < (1LL << 31)) {
        // p <= gp, so (p + 1) * S < 2^31 + S fits in 32 unsigned bits
        const uint32_t s = (uint32_t)S, a = (uint32_t)p * s / (uint32_t)gp;
        if ((w & 1) == 0) return a;
        const uint32_t e = (uint32_t)(p + 1) * s / (uint32_t)gp;
        return a + (e - a) * kDecEven64 / 64;
    }
    const long long a = (long long)p * S / gp;
    if ((w & 1) == 0) return a;
    const long long e = (long long)(p + 1) * S / gp;
    return a + (e - a) * kDecEven64 / 64;
}
// the wave whose range holds stage st (0 <= st < S)
__device__ __forceinline__ int dec_wave_of(long long st, long long S, int G) {
    const int gp = G >> 1;
    const int p = S * gp < (1LL << 31) ? (int)(((uint32_t)st + 1) * (uint32_t)gp - 1) / (int)S
                                        : (int)(((st + 1) * gp - 1) / S);
    return 2 * p + (st >= dec_range_start(2 * p + 1, S, G) ? 1 : 0);
}

template <int D, int DS, int QR>
struct StreamTile {
    static constexpr int BK = 32;                    // keys per stage
    static constexpr int TILE = BK * D;              // elements of K (or V) per stage
    static constexpr int QTILE = QR * D;             // query rows per stage
    static constexpr int STAGE = 2 * TILE + QTILE;
    static constexpr int LDS_BYTES = DS * STAGE * 2;
    static constexpr int IPT = BK * D / 8 / 64;      // load instructions per K (or V) tile
    static constexpr int QI = QR * D / 8 / 64;       // load instructions for the query rows
    static constexpr int LPS = 2 * IPT;              // K and V loads per stage
    static_assert(QI >= 1 && QR * D / 8 == QI * 64, "query rows must fill whole loads");
    static_assert((DS - 2) * LPS < 64, "vmcnt range");
};

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

// position in the stage sequence: sequence b (clamped length len, nb stages
// per row), row ri of that sequence's HK rows, stage j of that row
struct StreamCursor {
    int b, len, nb, ri, j;
};

template <int D, int DS, int QR>
__global__ __launch_bounds__(64) void decode_stream_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const int* __restrict__ seqlens, float* __restrict__ part_o, float* __restrict__ part_lse,
    int* __restrict__ meta, int B, int Hq, int Hkv, int Nmax, int nht, int G, float sl2, int cq,
    PageTable pt) {
    using T = StreamTile<D, DS, QR>;
    static_assert(DS <= 5, "wait_stages covers at most five stages");
    extern __shared__ __align__(16) uint16_t smem[];
    const int lane = threadIdx.x;
    const int n = lane & 31, hf = lane >> 5;
    const int g = Hq / Hkv;
    const int HK = Hkv * nht;                    // rows per sequence
    const int TR = min(g, 32);                   // partial rows per slot
    const int w = blockIdx.x;
    auto clen = [&](int b) { return max(0, min(Nmax, seqlens[b])); };
    // the same for a wave-uniform b (a scalar load)
    auto clen_u = [&](int b) { return max(0, min(Nmax, seqlens[__builtin_amdgcn_readfirstlane(b)])); };

    // total stage count S; wave 0 records the exclusive prefix per sequence.
    // Lane l holds sequence b0 + l of the last chunk read (all of them when
    // B <= 64, so the search below needs no second pass over the lengths).
    int S = 0, len_l = 0, cnt_l = 0, incl_l = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
        const int b = b0 + lane;
        len_l = b < B ? clen(b) : 0;
        cnt_l = (len_l + T::BK - 1) / T::BK * HK;
        incl_l = wave_incl_scan(cnt_l, lane);
        if (w == 0 && b < B) meta[b] = S + incl_l - cnt_l;
        S += __shfl(incl_l, 63, 64);
    }
    S = __builtin_amdgcn_readfirstlane(S);
    if (w == 0 && lane == 0) meta[B] = S;
    const int s0 = (int)dec_range_start(w, S, G);
    const int s1 = (int)dec_range_start(w + 1, S, G);
    const int total = s1 - s0;
    if (total <= 0) return;

    // the sequence holding stage s0, and s0's offset inside it
    int b_st = 0, off = 0, len_st = 0;
    {
        int run = 0;
        for (int b0 = 0; b0 < B; b0 += 64) {
            if (B > 64) {
                const int b = b0 + lane;
                len_l = b < B ? clen(b) : 0;
                cnt_l = (len_l + T::BK - 1) / T::BK * HK;
                incl_l = wave_incl_scan(cnt_l, lane);
            }
            const int excl = run + incl_l - cnt_l;
            const unsigned long long m = __ballot(cnt_l > 0 && excl <= s0 && s0 < excl + cnt_l);
            if (m) {
                const int l = __ffsll((long long)m) - 1;
                b_st = b0 + l;
                off = s0 - __shfl(excl, l, 64);
                len_st = __shfl(len_l, l, 64);
                break;
            }
            run += __shfl(incl_l, 63, 64);
        }
    }
    StreamCursor start;
    start.b = __builtin_amdgcn_readfirstlane(b_st);
    start.len = __builtin_amdgcn_readfirstlane(len_st);
    start.nb = (start.len + T::BK - 1) / T::BK;
    off = __builtin_amdgcn_readfirstlane(off);
    start.ri = off / start.nb;
    start.j = off % start.nb;

    auto advance = [&](StreamCursor& c) {
        if (++c.j < c.nb) return;
        c.j = 0;
        if (++c.ri < HK) return;
        c.ri = 0;
        do {
            if (++c.b >= B) return;   // past the last stage; never used
            c.len = clen_u(c.b);
            c.nb = (c.len + T::BK - 1) / T::BK;
        } while (c.nb == 0);
    };

    // Stage k goes to ring slot k % DS.  The row's query rows come along with
    // its first stage in this wave (a row start, or the wave's first stage),
    // issued before the stage's K and V loads: loads complete in order, so a
    // wait that leaves only r stages' K and V loads in flight also covers
    // every query load older than them, and the wait counts stay constant.
    // Keys at or past the sequence end are read from its last row (their
    // scores are masked to -inf); query rows past the group read its last head.
    size_t last_pidx = ~(size_t)0;   // table slot of the page issued last
    int last_pg = 0;
    auto issue = [&](const StreamCursor& c, int k) {
        uint16_t* kt = smem + (k % DS) * T::STAGE;
        uint16_t* vt = kt + T::TILE;
        uint16_t* qt = vt + T::TILE;
        const int hk = c.ri / nht, ht = c.ri % nht;
        if (c.j == 0 || k == 0) {
#pragma unroll
            for (int i = 0; i < T::QI; ++i) {
                const int slot = i * 64 + lane;
                const int row = slot / (D / 8), pos = slot % (D / 8);
                const int head = min(ht * 32 + row, g - 1);
                const size_t gi = (size_t)(c.b * Hq + hk * g + head) * D + ((pos ^ swz<D>(row)) << 3);
                __builtin_amdgcn_global_load_lds(Q + gi, DEC_LDS_PTR(qt + i * 64 * 8), 16, 0, 0);
            }
        }
        const int key0 = c.j * T::BK;
        // the stage's 32 keys are consecutive rows from row0 of kbase/vbase: of the
        // sequence's contiguous cache, or of the one page that holds them all
        const uint16_t* kbase;
        const uint16_t* vbase;
        int row0;
        if (pt.table) {
            // consecutive stages of one page reuse its table entry (a scalar
            // load the stage's addresses wait on): +8% on 64-key pages
            const size_t pidx = (size_t)c.b * pt.max_pages + key0 / pt.page_size;
            if (pidx != last_pidx) {
                last_pidx = pidx;
                last_pg = min(max(pt.table[pidx], 0), pt.num_pages - 1);
            }
            const int pg = last_pg;
            kbase = K + ((size_t)pg * Hkv + hk) * pt.page_size * D;
            vbase = V + ((size_t)pg * Hkv + hk) * pt.page_size * D;
            row0 = key0 % pt.page_size;
        } else {
            kbase = K + (size_t)(c.b * Hkv + hk) * Nmax * D;
            vbase = V + (size_t)(c.b * Hkv + hk) * Nmax * D;
            row0 = key0;
        }
        // K and V are read once: non-temporal loads (the nt cache policy, aux
        // bit 1), which measured 11% faster than default-policy loads on the
        // decode workload (6.25 against 5.63 TB/s with cold caches)
#pragma unroll
        for (int i = 0; i < T::IPT; ++i) {
            const int slot = i * 64 + lane;
            const int row = slot / (D / 8), pos = slot % (D / 8);
            const size_t gi = (size_t)(row0 + min(row, c.len - 1 - key0)) * D + ((pos ^ swz<D>(row)) << 3);
            __builtin_amdgcn_global_load_lds(kbase + gi, DEC_LDS_PTR(kt + i * 64 * 8), 16, 0, kLoadNonTemporal);
            __builtin_amdgcn_global_load_lds(vbase + gi, DEC_LDS_PTR(vt + i * 64 * 8), 16, 0, kLoadNonTemporal);
        }
    };

    StreamCursor ic = start, cc = start;
    const int pro = min(DS - 1, total);
    for (int k = 0; k < pro; ++k) {
        issue(ic, k);
        advance(ic);
    }
    bf16x8 qf[D / 16];

    f32x16 ot[D / 32];
#pragma unroll
    for (int md = 0; md < D / 32; ++md) ot[md] = zero16();
    float m_run = kNegInf, l_run = 0.f;

    for (int k = 0; k < total; ++k) {
        // stage k has landed once at most min(DS-2, total-1-k) younger stages remain
        wait_stages<T::LPS, DS>(min(DS - 2, total - 1 - k));
        __builtin_amdgcn_sched_barrier(0);
        if (k + DS - 1 < total) {
            issue(ic, k + DS - 1);
            advance(ic);
        }
        const uint16_t* sK = smem + (k % DS) * T::STAGE;
        const uint16_t* sV = sK + T::TILE;
        const uint16_t* sQ = sV + T::TILE;
        const int key0 = cc.j * T::BK;
        const int k_end = cc.len;
        // Causal chunk (cq new tokens per query head, cq = 1 otherwise): row
        // rho of the group is token rho % cq, which sees the keys below
        // k_end - (cq - 1 - rho % cq).  Lane n holds row 32 ht + n.
        const int row_lim = k_end - (cq - 1) + min(cc.ri % nht * 32 + n, g - 1) % cq;
        if (cc.j == 0 || k == 0) {
            // Q^T operand of the row: lane (n, hf) takes query row min(n, QR-1)
            const int qr = min(n, QR - 1);
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                qf[kk] = *reinterpret_cast<const bf16x8*>(sQ + swz_off<D>(qr, kk * 2 + hf));
        }
        bf16x8 kf[D / 16];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) kf[kk] = frag_rows_swz<D>(sK, 0, kk * 16, lane);
        f32x16 sc = zero16();
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) sc = mfma32x32x16(kf[kk], qf[kk], sc);
        if (key0 + T::BK > k_end - (cq - 1)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = key0 + (i >> 2) * 8 + hf * 4 + (i & 3);
                sc[i] = key < row_lim ? sc[i] : kNegInf;
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

        if (cc.j == cc.nb - 1 || k == total - 1) {
            // partial of this row over the stages this wave saw: O / l, m + log l
            const int hk = cc.ri / nht, ht = cc.ri % nht;
            const int gh = ht * 32 + n;
            const float l_tot = pair_sum(l_run);
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            if (gh < g) {
                const size_t slot = (size_t)(cc.b * HK + cc.ri + w) * TR + n;
                float* po = part_o + slot * D;
#pragma unroll
                for (int md = 0; md < D / 32; ++md)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        *reinterpret_cast<f32x4*>(po + md * 32 + q4 * 8 + hf * 4) =
                            f32x4{ot[md][q4 * 4] * inv, ot[md][q4 * 4 + 1] * inv, ot[md][q4 * 4 + 2] * inv,
                                  ot[md][q4 * 4 + 3] * inv};
                if (hf == 0) part_lse[slot] = l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : kNegInf;
            }
            (void)hk;
#pragma unroll
            for (int md = 0; md < D / 32; ++md) ot[md] = zero16();
            m_run = kNegInf;
            l_run = 0.f;
        }
        advance(cc);
    }
}

// Merge the partials of each (sequence, query head): the row's stages
// [P, P + nb) were covered by waves wave_of(P) .. wave_of(P + nb - 1), where
// wave w owns [dec_range_start(w), dec_range_start(w + 1)); waves with an
// empty range wrote nothing.
template <int D>
__global__ __launch_bounds__(D) void decode_stream_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, const int* __restrict__ meta,
    const int* __restrict__ seqlens, uint16_t* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Hkv,
    int Nmax, int nht, int G) {
    const int hq = blockIdx.x, b = blockIdx.y;
    const int dcol = threadIdx.x;
    const int g = Hq / Hkv, HK = Hkv * nht, TR = min(g, 32);
    const int hk = hq / g, gh = hq % g, ht = gh / 32, hi = gh % 32;
    const int len = max(0, min(Nmax, seqlens[b]));
    const int nb = (len + 31) / 32;
    uint16_t* orow = O + (size_t)(b * Hq + hq) * D;
    if (nb == 0) {
        orow[dcol] = 0;
        if (dcol == 0) LSE[b * Hq + hq] = kNegInf;
        return;
    }
    const long long S = meta[B];
    const int r = b * HK + hk * nht + ht;
    const long long P = meta[b] + (long long)(hk * nht + ht) * nb;
    auto wave_of = [&](long long st) { return dec_wave_of(st, S, G); };
    auto start_of = [&](int wv) { return dec_range_start(wv, S, G); };
    const int wf = wave_of(P), wl = wave_of(P + nb - 1);
    // The pieces' logsumexps are fetched together (one per thread) into LDS,
    // a chunk at a time, and merged with a running maximum, so the loads of
    // the pieces do not wait on each other.
    constexpr int CH = 4 * D;
    __shared__ float s_lse[CH];
    float M = kNegInf, L = 0.f, acc = 0.f;
    for (int c0 = wf; c0 <= wl; c0 += CH) {
        const int nc = min(CH, wl - c0 + 1);
        __syncthreads();
        for (int t = dcol; t < nc; t += D) {
            const int wv = c0 + t;
            s_lse[t] = start_of(wv) < start_of(wv + 1) ? part_lse[(size_t)(r + wv) * TR + hi] : kNegInf;
        }
        __syncthreads();
        float cm = kNegInf;
        for (int t = 0; t < nc; ++t) cm = __builtin_fmaxf(cm, s_lse[t]);
        const float m_new = __builtin_fmaxf(M, cm);
        const float corr = M == kNegInf ? 0.f : exp2_fast((M - m_new) * kLog2e);
        L *= corr;
        acc *= corr;
        M = m_new;
#pragma unroll 4
        for (int t = 0; t < nc; ++t) {
            // a wave with no stages wrote nothing: weight 0, and its slot's
            // (unwritten) contents are discarded by the select
            const float l = s_lse[t];
            const float v = part_o[((size_t)(r + c0 + t) * TR + hi) * D + dcol];
            // a piece that saw no key of this row (lse = -inf) weighs 0, also
            // while every piece so far is empty (M = -inf)
            const float wt = l == kNegInf ? 0.f : exp2_fast((l - M) * kLog2e);
            L += wt;
            acc += l == kNegInf ? 0.f : wt * v;
        }
    }
    // a row that sees no key at all (a causal chunk longer than its sequence): O = 0, LSE = -inf
    orow[dcol] = f32_to_bf16_bits(L > 0.f ? acc / L : 0.f);
    if (dcol == 0) LSE[b * Hq + hq] = L > 0.f ? M + log2_fast(L) * kLn2 : kNegInf;
}

template <int D, int DS, int QR>
static hipError_t launch_decode_stream(const DecodeArgs& a, int nht) {
    using T = StreamTile<D, DS, QR>;
    constexpr auto kern = decode_stream_kernel<D, DS, QR>;
    hipError_t e = ensure_dynamic_lds<kern>(T::LDS_BYTES);
    if (e != hipSuccess) return e;
    int ncu = 0, lds = 0;
    if ((e = device_caps(&ncu, &lds)) != hipSuccess) return e;
    // as many one-wave workgroups as the LDS of all CUs holds at once
    const int per_cu = std::max(1, std::min(8, lds / T::LDS_BYTES));
    const int G = std::max(2, std::min(kDecodeMaxWaves, ncu * per_cu) & ~1);   // even (pairs)
    hipLaunchKernelGGL(kern, dim3(G), dim3(64), T::LDS_BYTES, (hipStream_t)a.stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, a.seqlens, a.part_o, a.part_lse, a.meta, a.B,
                       a.Hq, a.Hkv, a.Nmax, nht, G, a.scale * kLog2e, a.cq, a.pages);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(decode_stream_combine_kernel<D>, dim3(a.Hq, a.B), dim3(D), 0, (hipStream_t)a.stream,
                       a.part_o, a.part_lse, a.meta, a.seqlens, (uint16_t*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.Nmax,
                       nht, G);
    return hipGetLastError();
}

// query rows staged in LDS: the group size rounded up to whole loads, at most 32
template <int D>
static hipError_t launch_decode_t(const DecodeArgs& a) {
    const int g = a.Hq / a.Hkv;
    const int nht = (g + 31) / 32;
    constexpr int RPL = 64 * 8 / D;   // rows per load instruction
    const int rows = std::min(g, 32);
    // Ring stages per streaming wave: two, except at d = 128 with one load of
    // query rows per stage, where three (two stages in flight per wave, three
    // waves per CU instead of four) measured 2.6% faster on the grouped-query
    // decode workload.  Stages of 32 query rows measured 3% slower with three.
    // The paged decode measured 3% slower with three as well, and takes them
    // anyway: the same shape then gets the same work split, so its results
    // equal the contiguous decode's bit for bit.
    if (rows <= RPL) {
        if (D == 128) return launch_decode_stream<D, 3, RPL>(a, nht);
        return launch_decode_stream<D, 2, RPL>(a, nht);
    }
    if (rows <= 2 * RPL) return launch_decode_stream<D, 2, std::min(2 * RPL, 32)>(a, nht);
    if (rows <= 4 * RPL) return launch_decode_stream<D, 2, std::min(4 * RPL, 32)>(a, nht);
    return launch_decode_stream<D, 2, 32>(a, nht);
}

hipError_t launch_decode_bf16(const DecodeArgs& a) {
    return a.d == 64 ? launch_decode_t<64>(a) : launch_decode_t<128>(a);
}

}  // namespace fa
