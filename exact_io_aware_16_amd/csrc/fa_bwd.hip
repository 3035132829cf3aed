// Backward pass of exact attention on gfx950.
//
// Recomputation (thienlv.com glossary "Flash Attention Là Gì?", section "Ba Kỹ
// Thuật Chính", item 2): P is never stored by the forward pass; the backward
// rebuilds it tile by tile from Q, K and the saved row logsumexp,
// P_ij = exp(scale q_i.k_j - lse_i), and then applies the chain rule of
// O = P V, P = softmax(scale Q K^T):
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D) with D_i = dO_i . O_i,
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// MI355X mapping.  Two kernels on one stream, no atomics, so the result is
// bitwise reproducible:
//  1. bwd_dq (query owner, shaped like the forward pass): each wave owns 32
//     query rows; it first forms D_i = dO_i . O_i of its rows in float32 (and
//     writes D and lse_i log2 e for the second kernel); S^T = K Q^T and
//     dP^T = V dO^T put one query per lane, so lse_i and D_i are per-lane
//     scalars; dQ^T += K^T dS^T accumulates in registers.  K and V blocks
//     stream through a ring of LDS stages filled by direct-to-LDS loads; K is
//     read both row-wise and with transposing reads (ds_read_b64_tr_b16) from
//     the same XOR-swizzled tile.
//  2. bwd_dkdv (key owner): each wave owns 32 keys for the whole pass, K and V
//     rows sit in registers, and for every query head of the group and every
//     query block S = Q K^T and dP = dO V^T put one key per lane; then
//     dV^T += dO^T P and dK^T += Q^T dS accumulate in registers.  Q and dO
//     tiles and the rows' lse log2 e and D stream through an LDS ring the
//     same way.  Grouped heads are summed in registers.
// The key-owner kernel recomputes S and dP that the query-owner kernel also
// computes (7 matrix products instead of 5); that buys determinism and removes
// every atomic read-modify-write of dQ.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

namespace {

// Store one wave's 32 x D gradient tile, held in the 32x32 MFMA accumulator
// layout (lane (n, hf): row n, columns md*32 + 8(i/4) + 4hf + i%4 of acc[md][i]),
// times `mul`, as whole 128-byte row segments.  Stored directly each
// instruction would write 16 (fp32) or 8 (bf16) bytes of 32 rows, partial
// lines that wait dirty in L2 for the write-back at kernel end.  Here each
// 128-byte column band of the tile is staged in the wave's 4 KB of LDS (row r,
// 16-byte chunk c at chunk c ^ (r mod 8)), read back by rows and written 16
// bytes per lane, 8 complete segments per instruction, with streaming stores.
// Rows r >= nrows are not written.  The wave's LDS operations complete in
// order, so a band's writes never overtake the previous band's reads.
template <int D, typename G>
__device__ __forceinline__ void store_tile_rows(G* base, int nrows, const f32x16* acc, float mul, uint8_t* stage,
                                                int lane) {
    constexpr int PW = 128 / (int)sizeof(G);   // columns per band
    const int n = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int p = 0; p < D / PW; ++p) {
#pragma unroll
        for (int mdl = 0; mdl < PW / 32; ++mdl) {
            const int md = p * (PW / 32) + mdl;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float a0 = acc[md][g * 4] * mul, a1 = acc[md][g * 4 + 1] * mul;
                const float a2 = acc[md][g * 4 + 2] * mul, a3 = acc[md][g * 4 + 3] * mul;
                if constexpr (sizeof(G) == 4) {
                    const int c = 2 * g + hf;
                    *reinterpret_cast<f32x4*>(stage + n * 128 + ((c ^ (n & 7)) << 4)) = f32x4{a0, a1, a2, a3};
                } else {
                    const int c = mdl * 4 + g;
                    *reinterpret_cast<u32x2*>(stage + n * 128 + ((c ^ (n & 7)) << 4) + hf * 8) =
                        u32x2{pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the band is in LDS
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = k * 8 + (lane >> 3), c = lane & 7;
            const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * 128 + ((c ^ (r & 7)) << 4));
            if (r < nrows)
                __builtin_nontemporal_store(
                    v, reinterpret_cast<u32x4*>(reinterpret_cast<char*>(base + (size_t)r * D) + p * 128 + c * 16));
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// 1. dQ, query owner
// ---------------------------------------------------------------------------
template <int D>
struct DqTile {
    static constexpr int BM = 128;                 // queries per workgroup (4 waves x 32)
    static constexpr int BN = 32;                  // keys per block
    static constexpr int TILE = BN * D;            // elements of one K (or V) block
    static constexpr int STAGE = 2 * TILE;         // K then V
    static constexpr int NS = 3;                   // ring stages
    static constexpr int LDS_BYTES = NS * STAGE * 2;
    static constexpr int IPW = TILE / 8 / 64 / 4;  // 16-byte load instructions per wave per tile
    static constexpr int LPS = 2 * IPW;
    static_assert(IPW >= 1 && TILE / 8 == IPW * 256, "tile must split evenly over the waves");
    static_assert((NS - 2) * LPS < 64, "vmcnt range");
};

template <int D, bool CAUSAL, typename G>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, float* __restrict__ delta,
    G* __restrict__ dQ, int Hq, int Hkv, int Nq, int Nk, int nqb, int BH, float sl2, float scale,
    const uint16_t* __restrict__ O, float* __restrict__ lse2_out) {
    using T = DqTile<D>;
    extern __shared__ __align__(16) uint16_t smem[];
    const int id = blockIdx.x;
    const int qb = CAUSAL ? (nqb - 1 - id / BH) : (id / BH);
    int b, h;
    group_major_head(id % BH, BH / Hq, Hq, Hkv, b, h);
    const int hk = h / (Hq / Hkv);
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int n = lane & 31, hf = lane >> 5;
    const int off = Nk - Nq;
    const int qw = qb * T::BM + wave * 32;
    const int qi = qw + n;
    const int qc = min(qi, Nq - 1);
    const size_t qrow = (size_t)(b * Hq + h) * Nq + qc;

    bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Q + qrow * D + kk * 16 + hf * 8));
        df[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(dO + qrow * D + kk * 16 + hf * 8));
    }
    const float lse_v = LSE[qrow];
    // rows with no visible key (lse = -inf) get P = 0
    const float lse2 = lse_v == kNegInf ? __builtin_huge_valf() : lse_v * kLog2e;
    // D = dO . O of this query row: O is read in the layout of the dO
    // fragments (this lane's half of the row), the halves meet across lanes
    // n and n + 32.  The row's D and lse2 (lse log2 e, +inf for a row that
    // saw no key so that P = exp2(s scale log2 e - lse2) = 0 there) go to the
    // workspace for the dK/dV kernel, which runs after this one.
    float dpart = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 of = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(O + qrow * D + kk * 16 + hf * 8));
#pragma unroll
        for (int e = 0; e < 8; ++e) dpart = __builtin_fmaf((float)of[e], (float)df[kk][e], dpart);
    }
    const float dlt = dpart + __shfl_xor(dpart, 32, 64);
    if (hf == 0 && qi < Nq) {
        delta[qrow] = dlt;
        lse2_out[qrow] = lse2;
    }

    const uint16_t* kb = K + (size_t)(b * Hkv + hk) * Nk * D;
    const uint16_t* vb = V + (size_t)(b * Hkv + hk) * Nk * D;
    // -D of this lane's query row in every element: the dP^T products
    // accumulate onto it, so dP - D costs no vector instruction per block
    f32x16 negd;
#pragma unroll
    for (int i = 0; i < 16; ++i) negd[i] = -dlt;
    int kv_end = Nk;
    if (CAUSAL) kv_end = min(Nk, qb * T::BM + T::BM + off);
    const int nblk = (kv_end + T::BN - 1) / T::BN;
    const int wave_end = CAUSAL ? min(Nk, qw + 32 + off) : Nk;

    f32x16 acc[D / 32];
#pragma unroll
    for (int md = 0; md < D / 32; ++md) acc[md] = zero16();

    // K and V blocks (dense, XOR-swizzled) travel global -> LDS with
    // direct-to-LDS loads into a ring of NS stages, NS-1 blocks ahead; K is
    // read row-wise for S^T = K Q^T and with transposing reads for
    // dQ^T += K^T dS^T.  Rows at or past kv_end read row kv_end - 1.
    auto issue = [&](int blk, int slot) {
        uint16_t* kt = smem + slot * T::STAGE;
        uint16_t* vt = kt + T::TILE;
#pragma unroll
        for (int i = 0; i < T::IPW; ++i) {
            const int sl = (wave * T::IPW + i) * 64 + lane;
            const int row = sl / (D / 8), pos = sl % (D / 8);
            const size_t gi = (size_t)min(blk * T::BN + row, kv_end - 1) * D + ((pos ^ swz<D>(row)) << 3);
            const int lds_off = (wave * T::IPW + i) * 64 * 8;
            __builtin_amdgcn_global_load_lds(kb + gi, LDS_PTR(kt + lds_off), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(vb + gi, LDS_PTR(vt + lds_off), 16, 0, 0);
        }
    };

#pragma unroll
    for (int st = 0; st < T::NS - 1; ++st) issue(st, st);
    // Block j uses ring slot j % NS; unrolled NS times so the slot is a
    // compile-time constant (LDS addresses: per-lane base plus immediates).
    auto block = [&](int j, auto slc) {
        constexpr int slot = decltype(slc)::value;
        const int key0 = j * T::BN;
        // this wave's loads of block j are done once at most NS-2 younger stages remain
        wait_vmcnt<(T::NS - 2) * T::LPS>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(j + T::NS - 1, (j + T::NS - 1) % T::NS);
        if (key0 < wave_end) {
            const uint16_t* sK = smem + slot * T::STAGE;
            const uint16_t* sV = sK + T::TILE;
            f32x16 s = zero16(), dp = negd;   // the products give dP^T - D directly
#pragma unroll
            for (int k0 = 0; k0 < D / 16; k0 += 4) {
                bf16x8 ka[4], va[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    ka[kk] = frag_rows_swz<D>(sK, 0, (k0 + kk) * 16, lane);
                    va[kk] = frag_rows_swz<D>(sV, 0, (k0 + kk) * 16, lane);
                }
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    s = mfma32x32x16(ka[kk], qf[k0 + kk], s);
                    dp = mfma32x32x16(va[kk], df[k0 + kk], dp);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // the 8 fragment reads
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);   // then the 8 MFMAs
            }
            // Whether this block needs the mask is the same for the whole wave;
            // taken through readfirstlane so that it is one scalar branch around
            // two copies of the loop (as a per-lane condition the compiler
            // guards every element with its own exec-masked branch).
            const bool need_mask = __builtin_amdgcn_readfirstlane(
                (int)(key0 + T::BN > kv_end || (CAUSAL && key0 + T::BN > qw + off)));
            auto form_ds = [&](auto masked) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float p = exp2_fast(__builtin_fmaf(s[i], sl2, -lse2));
                    if constexpr (decltype(masked)::value) {
                        const int key = key0 + (i >> 2) * 8 + hf * 4 + (i & 3);
                        const bool ok = key < kv_end && (!CAUSAL || key <= qi + off);
                        p = ok ? p : 0.f;
                    }
                    s[i] = p * dp[i];  // dS^T = P (dP - D)
                }
            };
            if (need_mask) form_ds(std::true_type{});
            else form_ds(std::false_type{});
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 db;
#pragma unroll
                for (int e = 0; e < 8; ++e) db[e] = (__bf16)s[ks * 8 + e];
#pragma unroll
                for (int md = 0; md < D / 32; ++md)
                    acc[md] = mfma32x32x16(frag_tr_swz<D>(sK, ks * 16, md * 32, lane), db, acc[md]);
            }
        }
    };
    for (int j0 = 0; j0 < nblk; j0 += T::NS) {
        static_for<0, T::NS>([&](auto slc) {
            if (j0 + decltype(slc)::value < nblk) block(j0 + decltype(slc)::value, slc);
        });
    }
    // the trailing look-ahead loads must land before the workgroup exits
    wait_vmcnt<0>();
    static_assert(4 * 4096 <= T::LDS_BYTES, "staging needs 4 KB per wave");
    __syncthreads();   // every wave is past its last ring read: the ring stages the output
    store_tile_rows<D>(dQ + ((size_t)(b * Hq + h) * Nq + qw) * D, Nq - qw, acc, scale,
                       reinterpret_cast<uint8_t*>(smem) + wave * 4096, lane);
}

// ---------------------------------------------------------------------------
// 2. dK, dV, key owner
// ---------------------------------------------------------------------------
// vector instructions placed after each MFMA of the next step in the
// software-pipelined dK/dV loop (d = 128)
constexpr int kDkvInterleave = 4;

template <int D>
struct DkvTile {
    static constexpr int BK = 128;                 // keys per workgroup (4 waves x 32)
    static constexpr int BQ = 32;                  // queries per step
    static constexpr int TILE = BQ * D;            // elements of one Q (or dO) tile
    static constexpr int AUX = 2 * BQ;             // floats per step: lse2[BQ], then delta[BQ]
    static constexpr int STAGE = 2 * TILE + 2 * AUX;   // uint16 elements
    static constexpr int NS = 3;                   // ring stages
    static constexpr int LDS_BYTES = NS * STAGE * 2;
    static constexpr int IPW = TILE / 8 / 64 / 4;  // 16-byte load instructions per wave per tile
    static constexpr int LPS = 2 * IPW + 1;        // per wave per stage (Q, dO, lse2/delta)
    static_assert(IPW >= 1 && TILE / 8 == IPW * 256, "tile must split evenly over the waves");
    static_assert((NS - 2) * LPS < 64, "vmcnt range");
};

// Key owner.  Q and dO tiles (BQ query rows each, dense and XOR-swizzled so
// that both 16-byte row reads and transposing reads are conflict-free) and
// the rows' lse2 and D travel global -> LDS with direct-to-LDS loads into a
// ring of NS stages, NS-1 steps ahead; one barrier per step.
template <int D, bool CAUSAL, typename G>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ delta,
    G* __restrict__ dK, G* __restrict__ dV, int Hq, int Hkv, int Nq, int Nk, int BHK, float sl2, float scale) {
    using T = DkvTile<D>;
    extern __shared__ __align__(16) uint16_t smem[];
    const int id = blockIdx.x;
    // Key blocks near the start see the most queries under the causal mask,
    // so launch slot id takes key block id / BHK: every (batch, K/V head)'s
    // heaviest block goes first.  The blocks of one (batch, head) are BHK
    // slots apart, so with BHK a multiple of 8 they share an XCD and its L2
    // copy of Q and dO.
    const int kblk = id / BHK;
    const int bhk = id % BHK;
    const int b = bhk / Hkv, hk = bhk % Hkv;
    const int g = Hq / Hkv;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int n = lane & 31, hf = lane >> 5;
    const int off = Nk - Nq;
    const int kw = kblk * T::BK + wave * 32;   // first key of this wave
    const int kj = kw + n;
    const int kc = min(kj, Nk - 1);
    const size_t krow = (size_t)(b * Hkv + hk) * Nk + kc;

    // K^T and V^T as the B operands: lane (n, hf) holds key kw + n
    bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        kf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(K + krow * D + kk * 16 + hf * 8));
        vf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(V + krow * D + kk * 16 + hf * 8));
    }

    f32x16 dv[D / 32], dk[D / 32];
#pragma unroll
    for (int md = 0; md < D / 32; ++md) {
        dv[md] = zero16();
        dk[md] = zero16();
    }

    // first query that sees any key of this workgroup / wave
    const int q_begin = CAUSAL ? max(0, kblk * T::BK - off) : 0;
    const int qb0 = q_begin / T::BQ;
    const int nqblk = (Nq + T::BQ - 1) / T::BQ - qb0;
    const int total = g * nqblk;   // (head, query block) steps
    const int wave_q_begin = CAUSAL ? max(0, kw - off) : 0;

    // step -> (query head, first query row).  Each head's query blocks are
    // taken last first, so the workgroups of one K/V head, which start
    // together (heaviest key blocks first) and share an XCD, stream the same
    // Q and dO tiles at the same time instead of each from its own causal
    // start, and read them from that XCD's L2.
    auto step_rows = [&](int step, size_t& base, int& q0) {
        const int hq = hk * g + step / nqblk;
        q0 = (qb0 + nqblk - 1 - step % nqblk) * T::BQ;   // last query block first
        base = (size_t)(b * Hq + hq) * Nq;
    };
    // this wave's share of step `step` into ring slot `slot` (steps past the
    // end reload the last one, rows past Nq reload row Nq - 1: the number of
    // loads per step is fixed and every address is valid)
    auto issue = [&](int step, int slot) {
        size_t base;
        int q0;
        step_rows(min(step, total - 1), base, q0);
        uint16_t* tq = smem + slot * T::STAGE;
        uint16_t* tdo = tq + T::TILE;
        uint16_t* taux = tdo + T::TILE;
#pragma unroll
        for (int i = 0; i < T::IPW; ++i) {
            const int sl = (wave * T::IPW + i) * 64 + lane;
            const int row = sl / (D / 8), pos = sl % (D / 8);
            const size_t gi = (base + min(q0 + row, Nq - 1)) * D + ((pos ^ swz<D>(row)) << 3);
            const int lds_off = (wave * T::IPW + i) * 64 * 8;
            __builtin_amdgcn_global_load_lds(Q + gi, LDS_PTR(tq + lds_off), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(dO + gi, LDS_PTR(tdo + lds_off), 16, 0, 0);
        }
        // lanes 0..BQ-1: lse2 of the step's rows, lanes BQ..2BQ-1: D (every
        // wave writes the same 256 bytes, which keeps the per-wave count equal)
        const int r = min(q0 + (lane % T::BQ), Nq - 1);
        const float* src = lane < T::BQ ? lse2 + base + r : delta + base + r;
        __builtin_amdgcn_global_load_lds(src, LDS_PTR(taux), 4, 0, 0);
    };

    if (total > 0) {
#pragma unroll
        for (int st = 0; st < T::NS - 1; ++st) issue(st, st);
    }
    // Step stp uses ring slot stp % NS; the loop is unrolled NS times so the
    // slot is a compile-time constant (LDS addresses: per-lane base plus
    // immediate offsets).
    auto step = [&](int stp, auto slc) {
        constexpr int slot = decltype(slc)::value;
        // this wave's loads of step stp are done once at most NS-2 younger stages remain
        wait_vmcnt<(T::NS - 2) * T::LPS>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(stp + T::NS - 1, (stp + T::NS - 1) % T::NS);
        size_t base_unused;
        int q0;
        step_rows(stp, base_unused, q0);
        if (q0 + T::BQ > wave_q_begin && kw < Nk) {
            const uint16_t* sQ = smem + slot * T::STAGE;
            const uint16_t* sdO = sQ + T::TILE;
            const float* sL = reinterpret_cast<const float*>(sdO + T::TILE);
            const float* sD = sL + T::BQ;
            // S = Q K^T, dP = dO V^T: one key per lane, 16 query rows per lane
            // fragments are read four k-steps at a time, ahead of their MFMAs
            f32x16 sc = zero16(), dp = zero16();
#pragma unroll
            for (int k0 = 0; k0 < D / 16; k0 += 4) {
                bf16x8 qa[4], da[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    qa[kk] = frag_rows_swz<D>(sQ, 0, (k0 + kk) * 16, lane);
                    da[kk] = frag_rows_swz<D>(sdO, 0, (k0 + kk) * 16, lane);
                }
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    sc = mfma32x32x16(qa[kk], kf[k0 + kk], sc);
                    dp = mfma32x32x16(da[kk], vf[k0 + kk], dp);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // the 8 fragment reads
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);   // then the 8 MFMAs
            }
            // one scalar branch around two copies of the loop (see the dQ kernel)
            const bool need_mask = __builtin_amdgcn_readfirstlane(
                (int)(kw + 32 > Nk || q0 + T::BQ > Nq || (CAUSAL && kw + 31 > q0 + off)));
            auto form_p_ds = [&](auto masked) {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int r0 = gq * 8 + hf * 4;   // query rows r0..r0+3 of this step
                    const f32x4 l4 = *reinterpret_cast<const f32x4*>(sL + r0);
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(sD + r0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = gq * 4 + r;
                        float p = exp2_fast(__builtin_fmaf(sc[i], sl2, -l4[r]));
                        if constexpr (decltype(masked)::value) {
                            const int qi = q0 + r0 + r;
                            const bool ok = kj < Nk && qi < Nq && (!CAUSAL || kj <= qi + off);
                            p = ok ? p : 0.f;
                        }
                        sc[i] = p;
                        dp[i] = p * (dp[i] - d4[r]);   // dS
                    }
                }
            };
            if (need_mask) form_p_ds(std::true_type{});
            else form_p_ds(std::false_type{});
            // dV^T += dO^T P and dK^T += Q^T dS, transposing reads of the same tiles
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 pb, db;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pb[e] = (__bf16)sc[ks * 8 + e];
                    db[e] = (__bf16)dp[ks * 8 + e];
                }
#pragma unroll
                for (int md = 0; md < D / 32; ++md) {
                    dv[md] = mfma32x32x16(frag_tr_swz<D>(sdO, ks * 16, md * 32, lane), pb, dv[md]);
                    dk[md] = mfma32x32x16(frag_tr_swz<D>(sQ, ks * 16, md * 32, lane), db, dk[md]);
                }
            }
        }
    };
    // d = 128 only: at d = 64 the second S/dP buffer would halve the waves per SIMD
    constexpr bool kPipe = D >= 128;
    if constexpr (kPipe) {
    // Software-pipelined over steps: iteration stp forms P and dS of step stp
    // and, in the same basic block, issues the S and dP products of step
    // stp + 1 (independent of them), so the matrix cores run under the
    // exponentials; then the dV and dK products of step stp.  S and dP are
    // double-buffered; the ring still holds three steps (stp, stp + 1 read;
    // stp + 2 loading).  Steps that a wave does not see (causal) or past the
    // end still get their S/dP computed from valid (clamped) data and the
    // result is never used.
    static_assert(T::NS == 3, "the pipelined loop reads two ring stages while a third loads");
    auto sdp = [&](auto slc, f32x16& sc, f32x16& dp) {
        constexpr int slot = decltype(slc)::value;
        const uint16_t* sQ = smem + slot * T::STAGE;
        const uint16_t* sdO = sQ + T::TILE;
        sc = zero16();
        dp = zero16();
#pragma unroll
        for (int k0 = 0; k0 < D / 16; k0 += 4) {
            bf16x8 qa[4], da[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                qa[kk] = frag_rows_swz<D>(sQ, 0, (k0 + kk) * 16, lane);
                da[kk] = frag_rows_swz<D>(sdO, 0, (k0 + kk) * 16, lane);
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                sc = mfma32x32x16(qa[kk], kf[k0 + kk], sc);
                dp = mfma32x32x16(da[kk], vf[k0 + kk], dp);
            }
        }
    };
    auto active = [&](int stp) {
        size_t base_unused;
        int q0;
        step_rows(stp, base_unused, q0);
        return q0 + T::BQ > wave_q_begin && kw < Nk;
    };
    f32x16 scb[2], dpb[2];
    if (total > 0) {
        // step 0's loads are done once only step 1's may still fly
        wait_vmcnt<T::LPS>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        sdp(std::integral_constant<int, 0>{}, scb[0], dpb[0]);
    }
    auto iteration = [&](int stp, auto u) {
        constexpr int U = decltype(u)::value;
        constexpr int cur = U % 3, nxt = (U + 1) % 3, bc = U % 2, bn = 1 - U % 2;
        // step stp + 1's loads (the only ones in flight) are done
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(stp + 2, (U + 2) % 3);
        auto next = [&]() { sdp(std::integral_constant<int, nxt>{}, scb[bn], dpb[bn]); };
        if (!active(stp)) {
            next();
            return;
        }
        size_t base_unused;
        int q0;
        step_rows(stp, base_unused, q0);
        const uint16_t* sQ = smem + cur * T::STAGE;
        const uint16_t* sdO = sQ + T::TILE;
        const float* sL = reinterpret_cast<const float*>(sdO + T::TILE);
        const float* sD = sL + T::BQ;
        f32x16& sc = scb[bc];
        f32x16& dp = dpb[bc];
        const bool need_mask = __builtin_amdgcn_readfirstlane(
            (int)(kw + 32 > Nk || q0 + T::BQ > Nq || (CAUSAL && kw + 31 > q0 + off)));
        auto form_p_ds = [&](auto masked) {
            next();
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int r0 = gq * 8 + hf * 4;
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(sL + r0);
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(sD + r0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = gq * 4 + r;
                    float p = exp2_fast(__builtin_fmaf(sc[i], sl2, -l4[r]));
                    if constexpr (decltype(masked)::value) {
                        const int qi = q0 + r0 + r;
                        const bool ok = kj < Nk && qi < Nq && (!CAUSAL || kj <= qi + off);
                        p = ok ? p : 0.f;
                    }
                    sc[i] = p;
                    dp[i] = p * (dp[i] - d4[r]);
                }
            }
            // interleave: the next step's fragment reads, then each of its
            // MFMAs followed by a few of this step's vector instructions
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, kDkvInterleave, 0);
                }
            }
        };
        if (need_mask) form_p_ds(std::true_type{});
        else form_p_ds(std::false_type{});
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 pb, db;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pb[e] = (__bf16)sc[ks * 8 + e];
                db[e] = (__bf16)dp[ks * 8 + e];
            }
#pragma unroll
            for (int md = 0; md < D / 32; ++md) {
                dv[md] = mfma32x32x16(frag_tr_swz<D>(sdO, ks * 16, md * 32, lane), pb, dv[md]);
                dk[md] = mfma32x32x16(frag_tr_swz<D>(sQ, ks * 16, md * 32, lane), db, dk[md]);
            }
        }
    };
    for (int s0 = 0; s0 < total; s0 += 6) {
        static_for<0, 6>([&](auto u) {
            if (s0 + decltype(u)::value < total) iteration(s0 + decltype(u)::value, u);
        });
    }
    } else {
    for (int s0 = 0; s0 < total; s0 += T::NS) {
        static_for<0, T::NS>([&](auto slc) {
            if (s0 + decltype(slc)::value < total) step(s0 + decltype(slc)::value, slc);
        });
    }
    }
    // the trailing look-ahead loads must land before the workgroup exits
    wait_vmcnt<0>();
    static_assert(4 * 4096 <= T::LDS_BYTES, "staging needs 4 KB per wave");
    __syncthreads();   // every wave is past its last ring read: the ring stages the output
    const size_t o = ((size_t)(b * Hkv + hk) * Nk + kw) * D;
    uint8_t* stage = reinterpret_cast<uint8_t*>(smem) + wave * 4096;
    store_tile_rows<D>(dK + o, Nk - kw, dk, scale, stage, lane);
    store_tile_rows<D>(dV + o, Nk - kw, dv, 1.f, stage, lane);
}

// ---------------------------------------------------------------------------
// float32 backward on the vector ALUs, four lanes per row (d/4 columns each)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_f32_kernel(const float* __restrict__ O, const float* __restrict__ dO,
                                                            float* __restrict__ delta, int rows) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    const int row = t >> 2, part = t & 3;
    float acc = 0.f;
    if (row < rows) {
        const float* a = O + (size_t)row * D + part * (D / 4);
        const float* c = dO + (size_t)row * D + part * (D / 4);
        for (int i = 0; i < D / 4; ++i) acc = __builtin_fmaf(a[i], c[i], acc);
    }
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    if (row < rows && part == 0) delta[row] = acc;
}

template <int D>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                         const float* __restrict__ V, const float* __restrict__ dO,
                                                         const float* __restrict__ LSE,
                                                         const float* __restrict__ delta, float* __restrict__ dQ,
                                                         int Hq, int Hkv, int Nq, int Nk, int causal, float sl2,
                                                         float scale) {
    constexpr int DS = D / 4, BK = 32;
    __shared__ float sK[BK][D + 4];
    __shared__ float sV[BK][D + 4];
    const int b = blockIdx.z, h = blockIdx.y, hk = h / (Hq / Hkv);
    const int tid = threadIdx.x, row = tid >> 2, part = tid & 3;
    const int qi = blockIdx.x * 64 + row;
    const int off = Nk - Nq;
    const size_t qr = (size_t)(b * Hq + h) * Nq + min(qi, Nq - 1);
    // gradient sums run over up to g * N terms: accumulated in float64 so the
    // float32 path stays within a few ulps of the exact result
    float q[DS], d_o[DS];
    double dq[DS];
#pragma unroll
    for (int c = 0; c < DS; ++c) {
        q[c] = Q[qr * D + part * DS + c];
        d_o[c] = dO[qr * D + part * DS + c];
        dq[c] = 0.0;
    }
    const float l = LSE[qr];
    const float lse2 = l == kNegInf ? __builtin_huge_valf() : l * kLog2e;
    const float dl = delta[qr];
    const float* kb = K + (size_t)(b * Hkv + hk) * Nk * D;
    const float* vb = V + (size_t)(b * Hkv + hk) * Nk * D;
    int end = Nk;
    if (causal) end = min(Nk, blockIdx.x * 64 + 64 + off);
    for (int key0 = 0; key0 < end; key0 += BK) {
        __syncthreads();
        for (int e = tid; e < BK * D; e += 256) {
            const int r = e / D, c = e % D;
            const int key = min(key0 + r, Nk - 1);
            sK[r][c] = kb[(size_t)key * D + c];
            sV[r][c] = vb[(size_t)key * D + c];
        }
        __syncthreads();
        for (int j = 0; j < BK; ++j) {
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int c = 0; c < DS; ++c) {
                s = __builtin_fmaf(q[c], sK[j][part * DS + c], s);
                dp = __builtin_fmaf(d_o[c], sV[j][part * DS + c], dp);
            }
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            dp += __shfl_xor(dp, 1, 64);
            dp += __shfl_xor(dp, 2, 64);
            const int key = key0 + j;
            const bool ok = key < Nk && (!causal || key <= qi + off);
            const float p = ok ? exp2_fast(__builtin_fmaf(s, sl2, -lse2)) : 0.f;
            const float ds = p * (dp - dl);
#pragma unroll
            for (int c = 0; c < DS; ++c) dq[c] = __builtin_fma((double)ds, (double)sK[j][part * DS + c], dq[c]);
        }
    }
    if (qi < Nq) {
#pragma unroll
        for (int c = 0; c < DS; ++c) dQ[qr * D + part * DS + c] = (float)(dq[c] * scale);
    }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                           const float* __restrict__ V, const float* __restrict__ dO,
                                                           const float* __restrict__ LSE,
                                                           const float* __restrict__ delta, float* __restrict__ dK,
                                                           float* __restrict__ dV, int Hq, int Hkv, int Nq, int Nk,
                                                           int causal, float sl2, float scale) {
    constexpr int DS = D / 4, BQ = 32;
    __shared__ float sQ[BQ][D + 4];
    __shared__ float sdO[BQ][D + 4];
    __shared__ float sL[BQ], sD[BQ];
    const int b = blockIdx.z, hk = blockIdx.y, g = Hq / Hkv;
    const int tid = threadIdx.x, row = tid >> 2, part = tid & 3;
    const int kj = blockIdx.x * 64 + row;
    const int off = Nk - Nq;
    const size_t kr = (size_t)(b * Hkv + hk) * Nk + min(kj, Nk - 1);
    float k[DS], v[DS];
    double dk[DS], dv[DS];   // float64 sums over g * N query rows
#pragma unroll
    for (int c = 0; c < DS; ++c) {
        k[c] = K[kr * D + part * DS + c];
        v[c] = V[kr * D + part * DS + c];
        dk[c] = 0.0;
        dv[c] = 0.0;
    }
    const int q_begin = causal ? max(0, (int)blockIdx.x * 64 - off) : 0;
    for (int hq = hk * g; hq < hk * g + g; ++hq) {
        const size_t base = (size_t)(b * Hq + hq) * Nq;
        for (int q0 = (q_begin / BQ) * BQ; q0 < Nq; q0 += BQ) {
            __syncthreads();
            for (int e = tid; e < BQ * D; e += 256) {
                const int r = e / D, c = e % D;
                const int qq = min(q0 + r, Nq - 1);
                sQ[r][c] = Q[(base + qq) * D + c];
                sdO[r][c] = dO[(base + qq) * D + c];
            }
            if (tid < BQ) {
                const int qq = min(q0 + tid, Nq - 1);
                const float l = LSE[base + qq];
                sL[tid] = l == kNegInf ? __builtin_huge_valf() : l * kLog2e;
                sD[tid] = delta[base + qq];
            }
            __syncthreads();
            for (int i = 0; i < BQ; ++i) {
                float s = 0.f, dp = 0.f;
#pragma unroll
                for (int c = 0; c < DS; ++c) {
                    s = __builtin_fmaf(sQ[i][part * DS + c], k[c], s);
                    dp = __builtin_fmaf(sdO[i][part * DS + c], v[c], dp);
                }
                s += __shfl_xor(s, 1, 64);
                s += __shfl_xor(s, 2, 64);
                dp += __shfl_xor(dp, 1, 64);
                dp += __shfl_xor(dp, 2, 64);
                const int qi = q0 + i;
                const bool ok = qi < Nq && kj < Nk && (!causal || kj <= qi + off);
                const float p = ok ? exp2_fast(__builtin_fmaf(s, sl2, -sL[i])) : 0.f;
                const float ds = p * (dp - sD[i]);
#pragma unroll
                for (int c = 0; c < DS; ++c) {
                    dv[c] = __builtin_fma((double)p, (double)sdO[i][part * DS + c], dv[c]);
                    dk[c] = __builtin_fma((double)ds, (double)sQ[i][part * DS + c], dk[c]);
                }
            }
        }
    }
    if (kj < Nk) {
#pragma unroll
        for (int c = 0; c < DS; ++c) {
            dK[kr * D + part * DS + c] = (float)(dk[c] * scale);
            dV[kr * D + part * DS + c] = (float)dv[c];
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, typename G>
static hipError_t launch_bwd_bf16_t(const BwdArgs& a) {
    const hipStream_t s = (hipStream_t)a.stream;
    const int rows = a.B * a.Hq * a.Nq;
    float* lse2 = a.delta + rows;
    hipError_t e;
    const float sl2 = a.scale * kLog2e;
    {
        using T = DqTile<D>;
        const int nqb = (a.Nq + T::BM - 1) / T::BM;
        const int BH = a.B * a.Hq;
        constexpr auto kern = bwd_dq_kernel<D, CAUSAL, G>;
        if ((e = ensure_dynamic_lds<kern>(T::LDS_BYTES)) != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(nqb * BH), dim3(256), T::LDS_BYTES, s, (const uint16_t*)a.q,
                           (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dO, a.lse, a.delta,
                           (G*)a.dq, a.Hq, a.Hkv, a.Nq, a.Nk, nqb, BH, sl2, a.scale, (const uint16_t*)a.o, lse2);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        using T = DkvTile<D>;
        const int nkb = (a.Nk + T::BK - 1) / T::BK;
        constexpr auto kern = bwd_dkdv_kernel<D, CAUSAL, G>;
        if ((e = ensure_dynamic_lds<kern>(T::LDS_BYTES)) != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(nkb * a.B * a.Hkv), dim3(256), T::LDS_BYTES, s, (const uint16_t*)a.q,
                           (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dO, lse2, a.delta,
                           (G*)a.dk, (G*)a.dv, a.Hq, a.Hkv, a.Nq, a.Nk, a.B * a.Hkv, sl2, a.scale);
    }
    return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_bf16_d(const BwdArgs& a) {
    if (a.grad_bf16)
        return a.causal ? launch_bwd_bf16_t<D, true, uint16_t>(a) : launch_bwd_bf16_t<D, false, uint16_t>(a);
    return a.causal ? launch_bwd_bf16_t<D, true, float>(a) : launch_bwd_bf16_t<D, false, float>(a);
}

hipError_t launch_bwd_bf16(const BwdArgs& a) { return a.d == 64 ? launch_bwd_bf16_d<64>(a) : launch_bwd_bf16_d<128>(a); }

template <int D>
static hipError_t launch_bwd_f32_d(const BwdArgs& a) {
    const hipStream_t s = (hipStream_t)a.stream;
    const int rows = a.B * a.Hq * a.Nq;
    hipLaunchKernelGGL(bwd_delta_f32_kernel<D>, dim3((rows * 4 + 255) / 256), dim3(256), 0, s, (const float*)a.o,
                       (const float*)a.dO, a.delta, rows);
    const float sl2 = a.scale * kLog2e;
    hipLaunchKernelGGL(bwd_dq_f32_kernel<D>, dim3((a.Nq + 63) / 64, a.Hq, a.B), dim3(256), 0, s, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (const float*)a.dO, a.lse, a.delta, (float*)a.dq, a.Hq,
                       a.Hkv, a.Nq, a.Nk, a.causal, sl2, a.scale);
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel<D>, dim3((a.Nk + 63) / 64, a.Hkv, a.B), dim3(256), 0, s,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (const float*)a.dO, a.lse, a.delta,
                       (float*)a.dk, (float*)a.dv, a.Hq, a.Hkv, a.Nq, a.Nk, a.causal, sl2, a.scale);
    return hipGetLastError();
}

hipError_t launch_bwd_f32(const BwdArgs& a) {
    // float32 gradients only (bfloat16 ones are rejected by the ABI layer)
    return a.d == 64 ? launch_bwd_f32_d<64>(a) : launch_bwd_f32_d<128>(a);
}

}  // namespace fa
