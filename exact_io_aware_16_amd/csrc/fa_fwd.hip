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
// MI355X mapping (bf16 kernel, fwd_ring_kernel):
//  * one workgroup = NW waves of 32 query rows of one (batch, head); each wave
//    owns its rows for the whole pass;
//  * K/V blocks of 64 keys go global -> LDS with direct-to-LDS loads
//    (global_load_lds_dwordx4) into a ring of S stages, S-1 blocks ahead, into
//    dense tiles with an XOR swizzle that keeps both row reads and transposing
//    reads (ds_read_b64_tr_b16) free of bank conflicts;
//  * scores are computed transposed, S^T = K Q^T (32x32x16 bf16 MFMA, fp32
//    accumulate), so every lane owns one query column: the row max and row sum
//    are per-lane reductions plus one exchange with lane l^32;
//  * the output is accumulated transposed too, O^T += V^T P^T, with V^T read
//    straight from the row-major V tile by transposing LDS reads, so the
//    rescale by exp(m_old - m_new) is a per-lane scalar;
//  * the softmax runs in base 2 with scale*log2(e) folded into one FMA, and the
//    running max is raised lazily (only on a jump of 2^64);
//  * causal: key blocks past the workgroup's last visible key are never
//    loaded, blocks past a wave's last visible key are skipped by that wave,
//    and only blocks crossing the diagonal pay for the mask;
//  * workgroups are issued heaviest query block first, and the blocks of one
//    (batch, head) are BH launch slots apart, so with BH a multiple of 8 they
//    land on the same XCD and share its L2 copy of K and V.
#include "fa_device.h"
#include "fa_launch.h"

#include <algorithm>

namespace fa {

// Tile shapes of the bf16 ring kernel (measured on MI355X; see the launchers)
constexpr int kRingWaves64 = 4;    // waves per workgroup, d = 64
constexpr int kRingStages64 = 2;   // ring stages, d = 64
constexpr int kRingWaves128 = 8;   // waves per workgroup, d = 128
constexpr int kRingStages128 = 2;  // ring stages, d = 128
// V fragments requested before the exponentials (d = 64, one column tile)
constexpr int kRingVAhead64 = 4;
// workgroups per CU the d = 64 ring kernel is compiled for (caps its VGPRs)
constexpr int kRingWgPerCu64 = 2;

// Lazy rescaling headroom (log2 units): the running max is only raised when
// some score of a block exceeds it by more than 64, so probabilities up to
// 2^64 are accumulated against a stale max (fp32 and bf16 hold them; l and O
// stay far below 2^128).  O and l share that max, so the final O / l is
// unchanged up to rounding.  Every row sees key 0 in its first block, so the
// first block sets a finite max and later blocks raise it only on a jump of
// 2^64, which typical score distributions never reach: the test is one
// per-lane compare against the lane's own block max, and the exchange between
// the two lanes of a query row, the rescale and its branch are left to the
// rare block that fails it.
constexpr float kRescaleHeadroom = 64.0f;

// ---------------------------------------------------------------------------
// Ring variant: K/V blocks travel global -> LDS with direct-to-LDS loads
// (global_load_lds_dwordx4, no register staging) into a ring of S stages, so
// S-1 blocks are in flight while one is computed.  The block loop is bound by
// load latency otherwise: a block's compute is far shorter than a round trip
// to L2/HBM.  Tiles are dense and XOR-swizzled (see swz()).  Per block: wait
// for this wave's loads of the block (vmcnt), one barrier (all waves' loads
// landed, and everybody finished the block that the next load overwrites),
// issue the load S-1 blocks ahead, compute.
// ---------------------------------------------------------------------------
template <int D, int NW, int S, int NT>
struct RingTile {
    static constexpr int QW = 32 * NT;             // query rows per wave
    static constexpr int BM = QW * NW;             // query rows per workgroup
    static constexpr int BN = 64;                  // keys per block
    static constexpr int TILE = BN * D;            // elements of one K (or V) block
    static constexpr int STAGE = 2 * TILE;         // K then V
    static constexpr int LDS_BYTES = S * STAGE * 2;
    static constexpr int IPW = (BN * D / 8) / 64 / NW;   // load instructions per wave per tile
    static constexpr int LPS = 2 * IPW;                  // per wave per stage (K and V)
    static_assert(IPW >= 1 && (BN * D / 8) % (64 * NW) == 0, "tile must split evenly over the waves");
};

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// sched_group_barrier masks
constexpr int kSgMfma = 0x008, kSgDsRead = 0x100;

template <int D, int NW, int S, int NT, bool CAUSAL>
__device__ __forceinline__ void fwd_qblock_ring(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                                                float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk, int b,
                                                int h, int qb, float sl2, uint16_t* smem) {
    using T = RingTile<D, NW, S, NT>;
    const int hk = h / (Hq / Hkv);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int n = lane & 31, hf = lane >> 5;

    const uint16_t* qbase = Q + (size_t)(b * Hq + h) * Nq * D;
    const uint16_t* kbase = K + (size_t)(b * Hkv + hk) * Nk * D;
    const uint16_t* vbase = V + (size_t)(b * Hkv + hk) * Nk * D;

    const int off = Nk - Nq;
    const int qw = qb * T::BM + wave * T::QW;

    // Q^T as the B operand (column tile nt: query qw + 32 nt + n); rows past Nq
    // read row Nq - 1 and are never stored.
    bf16x8 qf[NT][D / 16];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const uint16_t* qrow = qbase + (size_t)min(qw + nt * 32 + n, Nq - 1) * D;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qf[nt][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + kk * 16 + hf * 8));
    }

    int kv_end = Nk;
    if (CAUSAL) kv_end = min(Nk, qb * T::BM + T::BM + off);
    const int nblk = (kv_end + T::BN - 1) / T::BN;
    const int wave_end = CAUSAL ? min(Nk, qw + T::QW + off) : Nk;
    const int mask_from = CAUSAL ? (qw + off) : Nk;

    // Issue this wave's share of block `blk` into stage `st` (rows clamped to
    // kv_end - 1: always in bounds).  Lane l of load i writes slot
    // (wave*IPW + i)*64 + l of the tile: row = slot / (D/8), swizzled chunk
    // slot % (D/8), i.e. global chunk (slot % (D/8)) ^ swz(row).
    auto issue = [&](int blk, int st) {
        uint16_t* kt = smem + st * T::STAGE;
        uint16_t* vt = kt + T::TILE;
#pragma unroll
        for (int i = 0; i < T::IPW; ++i) {
            const int slot = (wave * T::IPW + i) * 64 + lane;
            const int row = slot / (D / 8), pos = slot % (D / 8);
            const size_t g = (size_t)min(blk * T::BN + row, kv_end - 1) * D + ((pos ^ swz<D>(row)) << 3);
            const int lds_off = (wave * T::IPW + i) * 64 * 8;   // elements; wave-uniform
            __builtin_amdgcn_global_load_lds(kbase + g, LDS_PTR(kt + lds_off), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(vbase + g, LDS_PTR(vt + lds_off), 16, 0, 0);
        }
    };

    f32x16 ot[NT][D / 32];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int md = 0; md < D / 32; ++md) ot[nt][md] = zero16();
    float m_run[NT], l_run[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        m_run[nt] = kNegInf;
        l_run[nt] = 0.f;
    }
    // row sums on the matrix cores: lacc[nt][0] / [1] of lane j < 16 hold the
    // running sums of queries j and j + 16 of column tile nt
    // (d = 64 only: no gain measured at d = 128)
    constexpr bool kMfmaSum = D == 64;
    f32x4 lacc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) lacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bf16x8 sel = rowsum_selector(lane);

    // prologue: blocks 0 .. S-2 (always S-1 stages issued, so the wait count is static)
#pragma unroll
    for (int st = 0; st < S - 1; ++st) issue(st, st);

    // Block j uses ring stage j % S.  The loop is unrolled S times so that the
    // stage is a compile-time constant: LDS fragment addresses become one
    // per-lane base plus immediate offsets (with a run-time stage the compiler
    // keeps a set of addresses per stage live).
    auto block = [&](int j, auto stc) {
        constexpr int st = decltype(stc)::value;
        // this wave's loads of block j are done once at most (S-2) stages remain outstanding
        wait_vmcnt<(S - 2) * T::LPS>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(j + S - 1, (j + S - 1) % S);

        const int key0 = j * T::BN;
        if (key0 < wave_end) {
            const uint16_t* sK = smem + st * T::STAGE;
            const uint16_t* sV = sK + T::TILE;
            // ---- S^T = K Q^T ----------------------------------------------------------
            f32x16 s[2][NT];
            if constexpr (D == 128 && NT == 1) {
                // the two 32-key halves' products alternate, so consecutive
                // MFMAs accumulate into different tiles; fragments are read
                // eight ahead of the products that use them
                bf16x8 kf[D / 16][2];
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) kf[kk][mt] = frag_rows_swz<D>(sK, mt * 32, kk * 16, lane);
                s[0][0] = zero16();
                s[1][0] = zero16();
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) s[mt][0] = mfma32x32x16(kf[kk][mt], qf[0][kk], s[mt][0]);
                constexpr int NR = 2 * (D / 16), AHEAD = 8;
                __builtin_amdgcn_sched_group_barrier(kSgDsRead, AHEAD, 0);
#pragma unroll
                for (int i = 0; i < NR - AHEAD; ++i) {
                    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(kSgMfma, AHEAD, 0);
            } else {
                // K fragments of a 32-key half are requested before its MFMAs, so LDS
                // latency is paid once per half; each fragment feeds NT MFMAs.
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    bf16x8 kf[D / 16];
#pragma unroll
                    for (int kk = 0; kk < D / 16; ++kk) kf[kk] = frag_rows_swz<D>(sK, mt * 32, kk * 16, lane);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) s[mt][nt] = zero16();
#pragma unroll
                    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) s[mt][nt] = mfma32x32x16(kf[kk], qf[nt][kk], s[mt][nt]);
                }
                // keep each half's fragment reads together, the second half's
                // issued while the first half's MFMAs run (left alone, the
                // compiler serialises every read with its MFMA to save registers)
                constexpr int NKH = D / 16;
                __builtin_amdgcn_sched_group_barrier(kSgDsRead, NKH, 0);
                __builtin_amdgcn_sched_group_barrier(kSgMfma, NKH * NT / 2, 0);
                __builtin_amdgcn_sched_group_barrier(kSgDsRead, NKH, 0);
                __builtin_amdgcn_sched_group_barrier(kSgMfma, NKH * NT * 3 / 2, 0);
            }
            // ---- mask (diagonal / tail blocks only) ---------------------------------------
            if (key0 + T::BN > mask_from || key0 + T::BN > kv_end) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int qi = qw + nt * 32 + n;
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int key = key0 + mt * 32 + (i >> 2) * 8 + hf * 4 + (i & 3);
                            const bool ok = key < kv_end && (!CAUSAL || key <= qi + off);
                            s[mt][nt][i] = ok ? s[mt][nt][i] : kNegInf;
                        }
                }
            }
            // ---- row max, lazy rescale ------------------------------------------------------
            float mx[NT];   // this lane's block max (log2 units); lanes n and n + 32 share a row
            bool grow = false;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                float m0 = kNegInf, m1 = kNegInf;
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    m0 = max3f(m0, s[0][nt][i], s[0][nt][i + 1]);
                    m1 = max3f(m1, s[1][nt][i], s[1][nt][i + 1]);
                }
                mx[nt] = __builtin_fmaxf(m0, m1) * sl2;
                grow |= !(mx[nt] <= m_run[nt] + kRescaleHeadroom);
            }
            if (!wave_all(!grow)) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const float m_new = __builtin_fmaxf(m_run[nt], pair_max(mx[nt]));
                    const float corr = (m_new == kNegInf) ? 1.f : exp2_fast(m_run[nt] - m_new);
                    if constexpr (kMfmaSum) {
                        const float corr_hi = __int_as_float(
                            __builtin_amdgcn_ds_bpermute(((lane + 16) & 63) << 2, __float_as_int(corr)));
                        lacc[nt][0] *= corr;
                        lacc[nt][1] *= corr_hi;
                    } else {
                        l_run[nt] *= corr;
                    }
#pragma unroll
                    for (int md = 0; md < D / 32; ++md)
#pragma unroll
                        for (int i = 0; i < 16; ++i) ot[nt][md][i] *= corr;
                    m_run[nt] = m_new;
                }
            }
            // V fragments of the first key groups are requested before the
            // exponentials so their latency hides behind the vector work.
            constexpr int VH = (D * NT == 64) ? kRingVAhead64 : 1;
            bf16x8 vf[VH][D / 32];
#pragma unroll
            for (int ks = 0; ks < VH; ++ks)
#pragma unroll
                for (int md = 0; md < D / 32; ++md) vf[ks][md] = frag_tr_swz<D>(sV, ks * 16, md * 32, lane);
            // ---- P = exp2(s*scale*log2e - m) in bf16, row sums ------------------------------
            bf16x8 pb[NT][T::BN / 16];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float m_use = (m_run[nt] == kNegInf) ? 0.f : m_run[nt];
                float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int i = 0; i < 16; i += 2) {
                        const float p0 = exp2_fast(__builtin_fmaf(s[mt][nt][i], sl2, -m_use));
                        const float p1 = exp2_fast(__builtin_fmaf(s[mt][nt][i + 1], sl2, -m_use));
                        ps0 += p0;
                        ps1 += p1;
                        pb[nt][mt * 2 + (i >> 3)][i & 7] = (__bf16)p0;
                        pb[nt][mt * 2 + (i >> 3)][(i & 7) + 1] = (__bf16)p1;
                    }
                if constexpr (!kMfmaSum) l_run[nt] += ps0 + ps1;
            }
            // ---- O^T += V^T P^T -------------------------------------------------------------
#pragma unroll
            for (int ks = 0; ks < T::BN / 16; ++ks) {
                bf16x8 va[D / 32];
#pragma unroll
                for (int md = 0; md < D / 32; ++md)
                    va[md] = ks < VH ? vf[ks < VH ? ks : 0][md] : frag_tr_swz<D>(sV, ks * 16, md * 32, lane);
#pragma unroll
                for (int md = 0; md < D / 32; ++md)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) ot[nt][md] = mfma32x32x16(va[md], pb[nt][ks], ot[nt][md]);
                if constexpr (kMfmaSum) {
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) lacc[nt] = mfma16x16x32(sel, pb[nt][ks], lacc[nt]);
                }
            }
        }
    };
    for (int j0 = 0; j0 < nblk; j0 += S) {
        static_for<0, S>([&](auto stc) {
            if (j0 + decltype(stc)::value < nblk) block(j0 + decltype(stc)::value, stc);
        });
    }
    // drain the ring's trailing loads before the workgroup's LDS is reused
    wait_vmcnt<0>();
    // every wave is past its last ring read and its loads have landed: the
    // ring becomes the staging area of the output tiles
    static_assert(NW * NT * 32 * D * 2 <= T::LDS_BYTES, "output tiles must fit in the ring");
    __syncthreads();

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int qi = qw + nt * 32 + n;
        float l_tot;
        if constexpr (kMfmaSum) {
            // query n's sum sits in lane n & 15, element n >> 4
            const float a0 = __int_as_float(__builtin_amdgcn_ds_bpermute((n & 15) << 2, __float_as_int(lacc[nt][0])));
            const float a1 = __int_as_float(__builtin_amdgcn_ds_bpermute((n & 15) << 2, __float_as_int(lacc[nt][1])));
            l_tot = n < 16 ? a0 : a1;
        } else {
            l_tot = pair_sum(l_run[nt]);
        }
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        {
            // O rows through LDS: the accumulator layout gives each lane 8-byte
            // pieces of 32 different rows, so stored directly every row is
            // written in sixteen 8-byte parts by eight instructions.  Staged
            // in this wave's own part of the ring (row q, 16-byte chunk c at
            // chunk c ^ (q mod chunks-per-row)), the rows are read back whole
            // and written as 16 bytes per lane, 64 / (D/8) complete rows per
            // instruction.
            constexpr int CPR = D / 8;      // 16-byte chunks per row
            constexpr int RPI = 64 / CPR;   // rows per store instruction
            uint16_t* so = smem + (wave * NT + nt) * 32 * D;
#pragma unroll
            for (int md = 0; md < D / 32; ++md)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c = md * 4 + g;
                    const uint32_t lo = pack_bf16x2(ot[nt][md][g * 4 + 0] * inv, ot[nt][md][g * 4 + 1] * inv);
                    const uint32_t hi = pack_bf16x2(ot[nt][md][g * 4 + 2] * inv, ot[nt][md][g * 4 + 3] * inv);
                    *reinterpret_cast<u32x2*>(so + n * D + ((c ^ (n & (CPR - 1))) << 3) + hf * 4) = u32x2{lo, hi};
                }
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's tile is in LDS
#pragma unroll
            for (int k = 0; k < 32 / RPI; ++k) {
                const int r = k * RPI + lane / CPR, c = lane % CPR;
                const u32x4 val = *reinterpret_cast<const u32x4*>(so + r * D + ((c ^ (r & (CPR - 1))) << 3));
                const int qr = qw + nt * 32 + r;
                if (qr < Nq) {
                    __builtin_nontemporal_store(
                        val, reinterpret_cast<u32x4*>(O + ((size_t)(b * Hq + h) * Nq + qr) * D + c * 8));
                }
            }
            if (qi < Nq && hf == 0) {
                const float lv = l_tot > 0.f ? (m_run[nt] + log2_fast(l_tot)) * kLn2 : kNegInf;
                __builtin_nontemporal_store(lv, LSE + (size_t)(b * Hq + h) * Nq + qi);
            }
        }
    }
}

template <int D, int NW, int S, int NT, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, ((NW == 4 && D * NT <= 128) ? kRingWgPerCu64 : 1)) void fwd_ring_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk, int nqb, int BH,
    float sl2) {
    extern __shared__ __align__(16) uint16_t smem[];
    const int slot = blockIdx.x / BH;
    int b, h;
    group_major_head(blockIdx.x % BH, BH / Hq, Hq, Hkv, b, h);
    fwd_qblock_ring<D, NW, S, NT, CAUSAL>(Q, K, V, O, LSE, Hq, Hkv, Nq, Nk, b, h, CAUSAL ? nqb - 1 - slot : slot, sl2,
                                          smem);
}

// ---------------------------------------------------------------------------
// float32 forward: the same recurrence on the vector ALUs, four lanes per query
// row (each owns d/4 columns).  Also serves float32 decode through kv_lens.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ V, float* __restrict__ O,
                                                      float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk,
                                                      int causal, float sl2, const int* __restrict__ kv_lens,
                                                      PageTable pt) {
    constexpr int DS = D / 4;   // columns per lane
    constexpr int BK = 32;      // keys per LDS block
    __shared__ float sK[BK][D + 4];
    __shared__ float sV[BK][D + 4];

    const int b = blockIdx.z, h = blockIdx.y;
    const int hk = h / (Hq / Hkv);
    const int tid = threadIdx.x;
    const int row = tid >> 2, part = tid & 3;
    const int qi = blockIdx.x * 64 + row;

    int kv_end = Nk;
    if (kv_lens) kv_end = max(0, min(Nk, kv_lens[b]));
    // causal is bottom-right aligned to the sequence's own length
    const int off = kv_end - Nq;
    int wg_end = kv_end;
    if (causal) wg_end = min(kv_end, blockIdx.x * 64 + 64 + off);

    const float* qrow = Q + ((size_t)(b * Hq + h) * Nq + (qi < Nq ? qi : 0)) * D + part * DS;

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
            size_t off_k;   // element offset of (key, c) from K (and V)
            if (pt.table) {
                const int pg = key < kv_end ? min(max(pt.table[(size_t)b * pt.max_pages + key / pt.page_size], 0),
                                                  pt.num_pages - 1)
                                            : 0;
                off_k = (((size_t)pg * Hkv + hk) * pt.page_size + key % pt.page_size) * D + c;
            } else {
                off_k = ((size_t)(b * Hkv + hk) * Nk + key) * D + c;
            }
            sK[r][c] = key < kv_end ? K[off_k] : 0.f;
            sV[r][c] = key < kv_end ? V[off_k] : 0.f;
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
template <int D, int NW, int S, int NT, bool CAUSAL>
static hipError_t launch_fwd_ring_t(const FwdArgs& a) {
    using T = RingTile<D, NW, S, NT>;
    const int nqb = (a.Nq + T::BM - 1) / T::BM;
    const int BH = a.B * a.Hq;
    constexpr auto kern = fwd_ring_kernel<D, NW, S, NT, CAUSAL>;
    const hipError_t e = ensure_dynamic_lds<kern>(T::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(nqb * BH), dim3(NW * 64), T::LDS_BYTES, (hipStream_t)a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse,
                       a.Hq, a.Hkv, a.Nq, a.Nk, nqb, BH, a.scale * kLog2e);
    return hipGetLastError();
}

// d = 64 with two 32-query column tiles per wave: every K and V fragment read
// from LDS feeds two MFMAs, which pays once there are enough workgroups
// (workgroups of 256 queries, 2 per CU) to fill the chip past the causal tail;
// smaller grids keep one tile per wave (more, lighter workgroups).
static bool fwd64_two_tiles(const FwdArgs& a) {
    int ncu = 256, lds = 0;
    if (device_caps(&ncu, &lds) != hipSuccess) ncu = 256;
    using T2 = RingTile<64, kRingWaves64, kRingStages64, 2>;
    const long long wgs = (long long)((a.Nq + T2::BM - 1) / T2::BM) * a.B * a.Hq;
    return wgs >= (long long)(a.causal ? 4 : 2) * ncu;
}

hipError_t launch_fwd_bf16(const FwdArgs& a) {
    if (a.d == 64) {
        if (fwd64_two_tiles(a))
            return a.causal ? launch_fwd_ring_t<64, kRingWaves64, kRingStages64, 2, true>(a)
                            : launch_fwd_ring_t<64, kRingWaves64, kRingStages64, 2, false>(a);
        return a.causal ? launch_fwd_ring_t<64, kRingWaves64, kRingStages64, 1, true>(a)
                        : launch_fwd_ring_t<64, kRingWaves64, kRingStages64, 1, false>(a);
    }
    return a.causal ? launch_fwd_ring_t<128, kRingWaves128, kRingStages128, 1, true>(a)
                    : launch_fwd_ring_t<128, kRingWaves128, kRingStages128, 1, false>(a);
}

template <int D>
static hipError_t launch_fwd_f32_t(const FwdArgs& a, const int* kv_lens, const PageTable* pages) {
    dim3 grid((a.Nq + 63) / 64, a.Hq, a.B);
    hipLaunchKernelGGL(fwd_f32_kernel<D>, grid, dim3(256), 0, (hipStream_t)a.stream, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.Hq, a.Hkv, a.Nq, a.Nk,
                       a.causal, a.scale * kLog2e, kv_lens,
                       pages ? *pages : PageTable{nullptr, 0, 0, 0});
    return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdArgs& a, const int* kv_lens, const PageTable* pages) {
    return a.d == 64 ? launch_fwd_f32_t<64>(a, kv_lens, pages) : launch_fwd_f32_t<128>(a, kv_lens, pages);
}

}  // namespace fa
