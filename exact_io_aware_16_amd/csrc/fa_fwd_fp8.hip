// FP8 forward: exact attention of OCP FP8 E4M3 inputs with one descale factor
// per tensor (thienlv.com glossary "Flash Attention Là Gì?", section "Flash
// Attention 2 và 3", which names FP8 support as a FlashAttention-3 feature;
// the recurrence is the one of the bf16 forward: handsonai.io "DL101 chapter
// 9", section 3.3).
//
// Both products run on the FP8 matrix cores (v_mfma_f32_32x32x64_f8f6f4,
// 32 x 32 outputs over 64 k per instruction, fp32 accumulation):
//   * S^T = K Q^T: K fragments from a swizzled LDS tile (lane (m, h) takes bytes
//     32h .. 32h+31 of a 64-wide d chunk of key row m), Q fragments in
//     registers with the same byte order; which k the hardware pairs is then
//     immaterial, as A and B bytes at one (lane half, byte) position meet.
//   * O^T += V^T P^T: P is scaled by 2^8 and rounded to E4M3 (round to nearest
//     even) in the accumulator's own order: lane (n, h) holds the 32 keys
//     mt*32 + 8*(i/4) + 4h + i%4 (mt = 0, 1; i = 0..15), byte 16 mt + i.  The
//     V^T operand is gathered from the row-major V tile with four
//     ds_read_b64_tr_b8 per fragment so that byte b of lane (m, h) holds V of
//     that same key at column m: ds_read_b64_tr_b8 hands lane i of a 16-lane
//     group byte i % 8 of the chunks addressed by lanes 2j + i / 8 (j = 0..7),
//     so lanes 2j and 2j + 1 address key row K(h, 8r + j) at columns
//     c0 .. c0+7 and c0+8 .. c0+15.
// The 2^8 keeps weights down to 2^-17 of the row maximum out of the E4M3
// flush region and the largest weight (256) exact; it requires the running
// maximum to be exact (no lazy rescale: a stale maximum would let P exceed the
// E4M3 range), so the rescale runs whenever the maximum grows.  The row sum l
// adds the scaled weights before rounding; O = descale_v * O' / l.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kFp8Waves = 4;    // waves per workgroup (d = 64 and 128)
constexpr int kFp8Stages = 3;   // ring stages (d = 64 and 128)

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr float kPScaleLog2 = 8.f;   // P is rounded to E4M3 as 2^8 * P

template <int D, int NW, int S>
struct Fp8Tile {
    static constexpr int QW = 32;                 // query rows per wave
    static constexpr int BM = QW * NW;            // query rows per workgroup
    static constexpr int BN = 64;                 // keys per block
    static constexpr int CPR = D / 16;            // 16-byte chunks per row
    static constexpr int TILE = BN * D;           // bytes of one K (or V) block
    static constexpr int STAGE = 2 * TILE;
    static constexpr int LDS_BYTES = S * STAGE;
    static constexpr int IPW = BN * CPR / 64 / NW;   // load instructions per wave per tile
    static constexpr int LPS = 2 * IPW;
    static_assert(IPW >= 1 && BN * CPR % (64 * NW) == 0, "tile must split evenly over the waves");
};

// XOR swizzle of the 16-byte chunks of row r in a tile.  A row holds D bytes,
// so 256 / D rows share one 256-byte line of the 64 LDS banks.  Two read
// forms must be conflict-free: 16 lanes reading one chunk of 16 consecutive
// rows (the K fragments), and the transposing byte reads of the V^T gather,
// where 16 lanes read one chunk of rows {R..R+3, R+8..R+11} and the other 16
// lanes of the same pass the neighbouring chunk.  d = 128 (two rows a line):
// rows of one parity take the swizzle (r >> 1) & 7 with bits 0 and 1
// swapped, a bijection over 16 consecutive rows that also splits rows R + t
// and R + 8 + t across chunk pairs.  d = 64 (four rows a line): (r >> 2) & 3.
template <int D>
__device__ __forceinline__ int fp8_swz(int r) {
    if constexpr (D == 128) {
        const int i = (r >> 1) & 7;
        return ((i & 1) << 1) | ((i >> 1) & 1) | (i & 4);
    } else {
        return (r >> 2) & 3;
    }
}

// byte offset of 16-byte chunk c of row r in a tile
template <int D>
__device__ __forceinline__ int off8(int r, int c) {
    return r * D + ((c ^ fp8_swz<D>(r)) << 4);
}

__device__ __forceinline__ f32x16 mfma_f8(const v8i& a, const v8i& b, const f32x16& c) {
    // format 0 (E4M3) for both operands; scale operands 0 select the unscaled instruction
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// key held in byte b of lane half h of a P / V^T operand
__device__ __forceinline__ constexpr int pkey(int h, int b) {
    return (b >> 4) * 32 + ((b & 15) >> 2) * 8 + h * 4 + (b & 3);
}

template <int D, int NW, int S, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk, int nqb, int BH, float sl2,
    float descale_v) {
    using T = Fp8Tile<D, NW, S>;
    extern __shared__ __align__(16) uint8_t smem8[];
    const int slot = blockIdx.x / BH;
    int b, h;
    group_major_head(blockIdx.x % BH, BH / Hq, Hq, Hkv, b, h);
    const int qb = CAUSAL ? nqb - 1 - slot : slot;
    const int hk = h / (Hq / Hkv);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int n = lane & 31, hf = lane >> 5;

    const uint8_t* qbase = Q + (size_t)(b * Hq + h) * Nq * D;
    const uint8_t* kbase = K + (size_t)(b * Hkv + hk) * Nk * D;
    const uint8_t* vbase = V + (size_t)(b * Hkv + hk) * Nk * D;
    const int off = Nk - Nq;
    const int qw = qb * T::BM + wave * T::QW;

    // Q^T operand: lane (n, hf) holds bytes 32 hf .. 32 hf + 31 of each 64-wide
    // d chunk of query row qw + n (rows past Nq read row Nq - 1, never stored)
    v8i qf[D / 64];
    {
        const uint8_t* qrow = qbase + (size_t)min(qw + n, Nq - 1) * D;
#pragma unroll
        for (int kc = 0; kc < D / 64; ++kc) {
            const u32x4 lo = *reinterpret_cast<const u32x4*>(qrow + kc * 64 + hf * 32);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(qrow + kc * 64 + hf * 32 + 16);
            qf[kc] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
    }

    int kv_end = Nk;
    if (CAUSAL) kv_end = min(Nk, qb * T::BM + T::BM + off);
    const int nblk = (kv_end + T::BN - 1) / T::BN;
    const int wave_end = CAUSAL ? min(Nk, qw + T::QW + off) : Nk;
    const int mask_from = CAUSAL ? (qw + off) : Nk;

    // this wave's share of block blk into stage st; rows clamped to kv_end - 1
    auto issue = [&](int blk, int st) {
        uint8_t* kt = smem8 + st * T::STAGE;
        uint8_t* vt = kt + T::TILE;
#pragma unroll
        for (int i = 0; i < T::IPW; ++i) {
            const int sl = (wave * T::IPW + i) * 64 + lane;
            const int row = sl / T::CPR, pos = sl % T::CPR;
            const size_t g = (size_t)min(blk * T::BN + row, kv_end - 1) * D + ((pos ^ fp8_swz<D>(row)) << 4);
            const int lds_off = (wave * T::IPW + i) * 64 * 16;
            __builtin_amdgcn_global_load_lds(kbase + g, (__attribute__((address_space(3))) void*)(kt + lds_off), 16,
                                             0, 0);
            __builtin_amdgcn_global_load_lds(vbase + g, (__attribute__((address_space(3))) void*)(vt + lds_off), 16,
                                             0, 0);
        }
    };

    f32x16 ot[D / 32];
#pragma unroll
    for (int md = 0; md < D / 32; ++md) ot[md] = zero16();
    float m_run = kNegInf, l_run = 0.f;

#pragma unroll
    for (int st = 0; st < S - 1; ++st) issue(st, st);

    // lane-constant parts of the V^T gather: group g = lane / 16 picks the lane
    // half (g / 2) and the 16-column half of the 32-row tile (g % 2); lane i of
    // the group addresses key row pkey(h, 8r + i/2) at column half i % 2
    const int grp = lane >> 4, gi = lane & 15;
    const int vh = grp >> 1;
    const int vcol16 = grp & 1;

    auto block = [&](int j, auto stc) {
        constexpr int st = decltype(stc)::value;
        wait_vmcnt<(S - 2) * T::LPS>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(j + S - 1, (j + S - 1) % S);

        const int key0 = j * T::BN;
        if (key0 < wave_end) {
            const uint8_t* sK = smem8 + st * T::STAGE;
            const uint8_t* sV = sK + T::TILE;
            // ---- S^T = K Q^T (2 key tiles of 32) ----------------------------------------
            f32x16 s[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                s[mt] = zero16();
#pragma unroll
                for (int kc = 0; kc < D / 64; ++kc) {
                    const int r = mt * 32 + n;
                    const u32x4 lo = *reinterpret_cast<const u32x4*>(sK + off8<D>(r, kc * 4 + hf * 2));
                    const u32x4 hi = *reinterpret_cast<const u32x4*>(sK + off8<D>(r, kc * 4 + hf * 2 + 1));
                    const v8i kf = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                    s[mt] = mfma_f8(kf, qf[kc], s[mt]);
                }
            }
            // ---- mask (diagonal / tail blocks) --------------------------------------------
            if (key0 + T::BN > mask_from || key0 + T::BN > kv_end) {
                const int qi = qw + n;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = key0 + mt * 32 + (i >> 2) * 8 + hf * 4 + (i & 3);
                        const bool ok = key < kv_end && (!CAUSAL || key <= qi + off);
                        s[mt][i] = ok ? s[mt][i] : kNegInf;
                    }
            }
            // ---- row max; exact rescale whenever it grows ----------------------------------
            float m0 = kNegInf, m1 = kNegInf;
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                m0 = max3f(m0, s[0][i], s[0][i + 1]);
                m1 = max3f(m1, s[1][i], s[1][i + 1]);
            }
            const float mx = pair_max(__builtin_fmaxf(m0, m1)) * sl2;
            if (!wave_all(mx <= m_run)) {
                const float m_new = __builtin_fmaxf(m_run, mx);
                const float corr = (m_new == kNegInf) ? 1.f : exp2_fast(m_run - m_new);
                l_run *= corr;
#pragma unroll
                for (int md = 0; md < D / 32; ++md)
#pragma unroll
                    for (int i = 0; i < 16; ++i) ot[md][i] *= corr;
                m_run = m_new;
            }
            // ---- P' = 2^8 exp2(s sl2 - m) rounded to E4M3, packed in key order pkey(hf, .) ---
            const float m_use = ((m_run == kNegInf) ? 0.f : m_run) - kPScaleLog2;
            v8i pf;
            float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const int mt = w >> 2, i0 = (w & 3) * 4;
                const float p0 = exp2_fast(__builtin_fmaf(s[mt][i0], sl2, -m_use));
                const float p1 = exp2_fast(__builtin_fmaf(s[mt][i0 + 1], sl2, -m_use));
                const float p2 = exp2_fast(__builtin_fmaf(s[mt][i0 + 2], sl2, -m_use));
                const float p3 = exp2_fast(__builtin_fmaf(s[mt][i0 + 3], sl2, -m_use));
                ps0 += p0 + p2;
                ps1 += p1 + p3;
                int x = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
                x = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, x, true);
                pf[w] = x;
            }
            l_run += ps0 + ps1;
            // ---- O^T += V^T P'^T: V^T gathered with transposing byte reads ------------------
#pragma unroll
            for (int md = 0; md < D / 32; ++md) {
                const int c16 = md * 2 + vcol16;
                v8i vf;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = pkey(vh, 8 * r + (gi >> 1));
                    const uint8_t* p = sV + off8<D>(row, c16) + (gi & 1) * 8;
                    const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)p);
                    vf[2 * r] = x[0];
                    vf[2 * r + 1] = x[1];
                }
                ot[md] = mfma_f8(vf, pf, ot[md]);
            }
        }
    };
    for (int j0 = 0; j0 < nblk; j0 += S) {
        static_for<0, S>([&](auto stc) {
            if (j0 + decltype(stc)::value < nblk) block(j0 + decltype(stc)::value, stc);
        });
    }
    wait_vmcnt<0>();

    const int qi = qw + n;
    const float l_tot = pair_sum(l_run);
    const float inv = l_tot > 0.f ? descale_v / l_tot : 0.f;
    {
        // O rows staged through this wave's part of the idle ring and written
        // whole with streaming stores (16 bytes per lane, complete rows per
        // instruction), as in the bf16 forward
        static_assert(NW * 32 * D * 2 <= T::LDS_BYTES, "output tiles must fit in the ring");
        constexpr int OCPR = D / 8;      // 16-byte chunks per bf16 row
        constexpr int RPI = 64 / OCPR;   // rows per store instruction
        __syncthreads();                 // every wave is past its last ring read
        uint16_t* so = reinterpret_cast<uint16_t*>(smem8) + wave * 32 * D;
#pragma unroll
        for (int md = 0; md < D / 32; ++md)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = md * 4 + g;
                const uint32_t lo = pack_bf16x2(ot[md][g * 4 + 0] * inv, ot[md][g * 4 + 1] * inv);
                const uint32_t hi = pack_bf16x2(ot[md][g * 4 + 2] * inv, ot[md][g * 4 + 3] * inv);
                *reinterpret_cast<u32x2*>(so + n * D + ((c ^ (n & (OCPR - 1))) << 3) + hf * 4) = u32x2{lo, hi};
            }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
#pragma unroll
        for (int k = 0; k < 32 / RPI; ++k) {
            const int r = k * RPI + lane / OCPR, c = lane % OCPR;
            const u32x4 val = *reinterpret_cast<const u32x4*>(so + r * D + ((c ^ (r & (OCPR - 1))) << 3));
            if (qw + r < Nq)
                __builtin_nontemporal_store(
                    val, reinterpret_cast<u32x4*>(O + ((size_t)(b * Hq + h) * Nq + qw + r) * D + c * 8));
        }
        if (qi < Nq && hf == 0)
            __builtin_nontemporal_store(l_tot > 0.f ? (m_run + log2_fast(l_tot) - kPScaleLog2) * kLn2 : kNegInf,
                                        LSE + (size_t)(b * Hq + h) * Nq + qi);
    }
}

template <int D, int NW, int S, bool CAUSAL>
hipError_t launch_fp8_t(const Fp8Args& a) {
    using T = Fp8Tile<D, NW, S>;
    const int nqb = (a.Nq + T::BM - 1) / T::BM;
    const int BH = a.B * a.Hq;
    constexpr auto kern = fwd_fp8_kernel<D, NW, S, CAUSAL>;
    const hipError_t e = ensure_dynamic_lds<kern>(T::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(nqb * BH), dim3(NW * 64), T::LDS_BYTES, (hipStream_t)a.stream,
                       (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v, (uint16_t*)a.o, a.lse, a.Hq,
                       a.Hkv, a.Nq, a.Nk, nqb, BH, a.scale * a.descale_q * a.descale_k * kLog2e, a.descale_v);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Args& a) {
    if (a.d == 64)
        return a.causal ? launch_fp8_t<64, kFp8Waves, kFp8Stages, true>(a)
                        : launch_fp8_t<64, kFp8Waves, kFp8Stages, false>(a);
    return a.causal ? launch_fp8_t<128, kFp8Waves, kFp8Stages, true>(a)
                    : launch_fp8_t<128, kFp8Waves, kFp8Stages, false>(a);
}

}  // namespace fa
