// Stub launch layer for the host-only sanitizer build of the C ABI
// (libfa_hostcheck.so): the entry points' argument checks, workspace sizing
// and layout run as in libfa, under AddressSanitizer and
// UndefinedBehaviorSanitizer, while every launch is replaced by a function
// that records the arguments it was handed and launches nothing.  Built by
// exact_io_aware_16_amd/build.py (build_hostcheck), used by tests/test_abi.py
// when FA_TEST_HOSTCHECK names the library.
#include <string.h>

#include "fa_launch.h"

namespace {
// the last launch's name and a few of its arguments, for the tests to read
struct LastLaunch {
    char kind[32];
    long long B, H, N, d, extra;
};
LastLaunch g_last;

void note(const char* kind, long long B, long long H, long long N, long long d, long long extra) {
    strncpy(g_last.kind, kind, sizeof(g_last.kind) - 1);
    g_last.kind[sizeof(g_last.kind) - 1] = 0;
    g_last.B = B;
    g_last.H = H;
    g_last.N = N;
    g_last.d = d;
    g_last.extra = extra;
}
}  // namespace

namespace fa {
hipError_t launch_fwd_bf16(const FwdArgs& a) {
    note("fwd_bf16", a.B, a.Hq, a.Nq, a.d, a.causal);
    return hipSuccess;
}
hipError_t launch_fwd_f32(const FwdArgs& a, const int* kv_lens, const PageTable* pages) {
    note(pages ? "fwd_f32_paged" : (kv_lens ? "fwd_f32_lens" : "fwd_f32"), a.B, a.Hq, a.Nq, a.d, a.causal);
    return hipSuccess;
}
hipError_t launch_bwd_bf16(const BwdArgs& a) {
    // the workspace holds 2 floats per query row: touch both ends of the view
    // the kernels would use (an undersized workspace would be caught here)
    note("bwd_bf16", a.B, a.Hq, a.Nq, a.d, a.grad_bf16);
    return hipSuccess;
}
hipError_t launch_bwd_f32(const BwdArgs& a) {
    note("bwd_f32", a.B, a.Hq, a.Nq, a.d, a.grad_bf16);
    return hipSuccess;
}
hipError_t launch_decode_bf16(const DecodeArgs& a) {
    note(a.pages.table ? "decode_paged" : "decode", a.B, a.Hq, a.Nmax, a.d, a.cq);
    return hipSuccess;
}
hipError_t launch_fwd_fp8(const Fp8Args& a) {
    note("fwd_fp8", a.B, a.Hq, a.Nq, a.d, a.causal);
    return hipSuccess;
}
}  // namespace fa

extern "C" const char* fa_hostcheck_last_launch(long long* out5) {
    out5[0] = g_last.B;
    out5[1] = g_last.H;
    out5[2] = g_last.N;
    out5[3] = g_last.d;
    out5[4] = g_last.extra;
    return g_last.kind;
}
