// Internal launch interface between the C-ABI layer (fa_api.hip) and the
// kernel files.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

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
    float* delta;  // workspace: [B][Hq][Nq] float32
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
    float* part_o;    // workspace: [B][Hq][nsplit][d] float32
    float* part_lse;  // workspace: [B][Hq][nsplit] float32
    int nsplit;
    void* stream;
};

hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a, const int* kv_lens);
hipError_t launch_bwd_bf16(const BwdArgs& a);
hipError_t launch_bwd_f32(const BwdArgs& a);
hipError_t launch_decode_bf16(const DecodeArgs& a);

// Keys per decode split (one workgroup streams one split of one KV head).
constexpr int kDecodeSplit = 512;

}  // namespace fa
