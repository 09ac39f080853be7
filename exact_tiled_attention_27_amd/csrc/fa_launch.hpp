// fa_launch.hpp -- internal launcher interface between the C ABI (fa_api.cpp)
// and the kernels.  Arguments reach here already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
    const void *q, *k, *v;
    float *o, *lse;
    int B, Hq, Hkv, N, d;
    float scale;   // > 0
    float tau;     // rescale threshold in the base-2 exponent domain
    bool causal;
    int poly;      // exponentials on the FMA units: 0 none, 4 one in four, 1 all
    int window;    // causal sliding window in keys (0: none)
    int splits;    // key chunks per query tile (1: one pass, no partials)
    float *opart;  // splits > 1: partial O, [splits][B * Hq][N][d] fp32
    float *lpart;  // splits > 1: partial LSE, [splits][B * Hq][N] fp32
    hipStream_t stream;
};

struct BwdArgs {
    const void *q, *k, *v, *dout;
    const float *o, *lse;
    float *dq, *dk, *dv;
    float *delta;  // workspace: D_i = sum_c dO_ic O_ic, [B, Hq, N]
    float *lse2;   // workspace: LSE_i * log2(e), [B, Hq, N]
    int B, Hq, Hkv, N, d;
    float scale;
    bool causal, deterministic;
    int window;    // causal sliding window in keys (0: none)
    hipStream_t stream;
};

hipError_t launch_fwd(const FwdArgs &a);
hipError_t launch_bwd(const BwdArgs &a);

// Rescale threshold: log2(256) = 8 (conditional rescaling).
constexpr float kRescaleTau = 8.0f;

// Window value the kernels receive when there is none: wider than any
// sequence, and small enough that q0 + 256 - kNoWindow cannot overflow.
constexpr int kNoWindow = 1 << 30;

}  // namespace fa
