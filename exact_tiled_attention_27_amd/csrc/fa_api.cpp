// fa_api.cpp -- the C ABI declared in include/fa.h: argument validation,
// workspace layout and dispatch to the gfx950 kernels.  Nothing here touches
// the GPU before every argument has been checked.
#include "fa.h"
#include "fa_debug.h"

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <cstdint>

#include "fa_launch.hpp"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape and scale checks shared by forward and backward.
int check_common(int B, int Hq, int Hkv, int N, int d, float scale)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    // Largest element offset must fit the kernels' 64-bit indexing and the
    // 32-bit grid: B * Hq * ceil(N / 64) workgroups.
    const int64_t rows = (int64_t)B * Hq * N;
    if (rows > ((int64_t)1 << 40) || (int64_t)B * Hq * ((N + 63) / 64) > INT32_MAX) return FA_ERR_SHAPE;
    // One head's rows, N * d bf16 values, are addressed with 32-bit byte
    // offsets (the tile copies use buffer resources over a head).
    if ((int64_t)N * d * 2 >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
    return FA_OK;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Backward workspace rows: every head's rows padded to a multiple of 64.
size_t workspace_rows(int B, int Hq, int N) { return (size_t)B * Hq * (size_t)((N + 63) & ~63); }

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// FA_RESCALE_TAU overrides the rescale threshold (base-2 exponent units, a
// finite value >= 0; 0 rescales whenever the running maximum grows, the
// textbook online softmax).  Unset or invalid: log2(256) = 8.  Read on every
// call.
float rescale_tau()
{
    const char *e = std::getenv("FA_RESCALE_TAU");
    if (!e) return fa::kRescaleTau;
    char *end = nullptr;
    const float t = std::strtof(e, &end);
    if (end == e || *end != '\0' || !std::isfinite(t) || t < 0.f) return fa::kRescaleTau;
    return t;
}

// FA_WORKGROUP_ORDER=linear launches workgroups in plain head-major order
// instead of the XCD-grouped (and, causal, longest-first) order: a switch for
// measuring what that order gains.  Read on every call.
int linear_map()
{
    const char *e = std::getenv("FA_WORKGROUP_ORDER");
    return (e && std::strcmp(e, "linear") == 0) ? 1 : 0;
}

// FA_PAIR_PATH=memory makes the paired atomic mode hand its partials over
// with device-scope stores and loads even when both blocks of a pair run on
// one XCD (the path taken otherwise only for pairs split across XCDs): a
// switch for testing that path and measuring what the L2 path gains.  Read
// on every call.
int pair_memory()
{
    const char *e = std::getenv("FA_PAIR_PATH");
    return (e && std::strcmp(e, "memory") == 0) ? 1 : 0;
}

// FA_WAIT_TICKS replaces the longest wait of the ordered and paired modes
// for another workgroup (100 MHz wall-clock ticks, an integer >= 0; 0: any
// wait whose condition is not met at once gives up), so that tests can
// exercise the timeout path; unset or invalid: 2 s.  Read on every call.
long long wait_ticks()
{
    const char *e = std::getenv("FA_WAIT_TICKS");
    if (!e) return fa::kWaitTicks;
    char *end = nullptr;
    const long long t = std::strtoll(e, &end, 10);
    if (end == e || *end != '\0' || t < 0) return fa::kWaitTicks;
    return t;
}

bool valid_bwd_mode(int mode) { return mode >= FA_BWD_ATOMIC && mode <= FA_BWD_ATOMIC_PAIRED; }

// Backward workspace bytes for dQ mode `mode`: the D and LSE2 rows, then the
// ordered mode's counters, or the paired atomic mode's pair block and ring.
size_t bwd_bytes(int B, int Hq, int Hkv, int N, int d, int mode)
{
    const size_t rows_part = 2 * round256(workspace_rows(B, Hq, N) * sizeof(float));
    if (mode == FA_BWD_ORDERED) return rows_part + round256(fa::bwd_sync_words(B * Hq, N) * sizeof(int));
    if (mode == FA_BWD_ATOMIC_PAIRED)
        return rows_part + round256(fa::bwd_pair_words(B, Hkv, N) * sizeof(int)) +
               round256(fa::bwd_pair_ring_bytes(B, Hkv, N, d));
    return rows_part;
}

// FA_EXP2_POLY selects how many of the forward's exponentials run as the
// cubic polynomial on the FMA units: "1" all, "4" one in four, anything else
// (or unset) none.  Read on every call.
int exp2_poly_share()
{
    const char *e = std::getenv("FA_EXP2_POLY");
    if (!e) return 0;
    if (std::strcmp(e, "1") == 0) return 1;
    if (std::strcmp(e, "4") == 0) return 4;
    return 0;
}

// fa_fwd and fa_fwd_window: window 0 = none (then causal as given), else
// causal with that window (>= 1, checked by the caller).
int fwd_impl(const void *q, const void *k, const void *v, float *o, float *lse, int B, int Hq,
             int Hkv, int N, int d, float scale, int causal, int window, void *stream,
             const float *slopes = nullptr)
{
    if (!q || !k || !v || !o) return FA_ERR_NULL;
    int st = check_common(B, Hq, Hkv, N, d, scale);
    if (st != FA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        (lse && !aligned16(lse)))
        return FA_ERR_ALIGN;
    fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, scale, rescale_tau(), causal != 0,
                  slopes ? 0 : exp2_poly_share(), window < N ? window : 0, 1, nullptr, nullptr,
                  reinterpret_cast<hipStream_t>(stream), slopes, linear_map()};
    return hip_status(fa::launch_fwd(a));
}

// fa_bwd and fa_bwd_window: window as in fwd_impl; deterministic is the dQ
// mode (FA_BWD_ATOMIC, FA_BWD_SEPARATE, FA_BWD_ORDERED or
// FA_BWD_ATOMIC_PAIRED).
int bwd_impl(const void *q, const void *k, const void *v, const float *o, const float *lse,
             const void *dout, float *dq, float *dk, float *dv, int B, int Hq, int Hkv, int N,
             int d, float scale, int causal, int window, int deterministic, void *workspace,
             size_t workspace_bytes, void *stream, const float *slopes = nullptr)
{
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
    int st = check_common(B, Hq, Hkv, N, d, scale);
    if (st != FA_OK) return st;
    if (!valid_bwd_mode(deterministic)) return FA_ERR_SHAPE;
    const void *ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
    for (const void *p : ptrs)
        if (!aligned16(p)) return FA_ERR_ALIGN;
    const size_t need = bwd_bytes(B, Hq, Hkv, N, d, deterministic);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
    const int pair_slots = deterministic == FA_BWD_ATOMIC_PAIRED ? fa::kPairSlots : 0;
    const size_t rows = workspace_rows(B, Hq, N);
    char *ws = reinterpret_cast<char *>(workspace);
    float *delta = reinterpret_cast<float *>(ws);
    float *lse2 = reinterpret_cast<float *>(ws + round256(rows * sizeof(float)));
    char *after_rows = ws + 2 * round256(rows * sizeof(float));
    int *sync = deterministic == FA_BWD_ORDERED || pair_slots > 0
                    ? reinterpret_cast<int *>(after_rows)
                    : nullptr;
    float *xring = pair_slots > 0
                       ? reinterpret_cast<float *>(
                             after_rows +
                             round256(fa::bwd_pair_words(B, Hkv, N) * sizeof(int)))
                       : nullptr;
    static_assert(fa::kBwdAtomic == FA_BWD_ATOMIC && fa::kBwdSeparate == FA_BWD_SEPARATE &&
                      fa::kBwdOrdered == FA_BWD_ORDERED &&
                      fa::kBwdAtomicPaired == FA_BWD_ATOMIC_PAIRED,
                  "dQ mode values");
    fa::BwdArgs a{q, k, v, dout, o, lse, dq, dk, dv, delta, lse2, sync, B, Hq, Hkv, N, d, scale,
                  causal != 0, deterministic, window < N ? window : 0,
                  reinterpret_cast<hipStream_t>(stream), slopes, linear_map(), xring, pair_slots,
                  pair_memory(), wait_ticks()};
    return hip_status(fa::launch_bwd(a));
}

}  // namespace

extern "C" {

const char *fa_status_string(int status)
{
    switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: invalid B/Hq/Hkv/N, scale, window, split count or dQ mode";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dimension must be 64 or 128";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: pointers must be 16-byte aligned";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown fa_status";
    }
}

int fa_fwd(const void *q, const void *k, const void *v, float *o, float *lse, int B, int Hq,
           int Hkv, int N, int d, float scale, int causal, void *stream)
{
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, 0, stream);
}

int fa_fwd_window(const void *q, const void *k, const void *v, float *o, float *lse, int B,
                  int Hq, int Hkv, int N, int d, float scale, int window, void *stream)
{
    if (window < 1) return FA_ERR_SHAPE;
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, 1, window, stream);
}

size_t fa_fwd_splitkv_workspace_bytes(int B, int Hq, int Hkv, int N, int d, int num_splits)
{
    if (check_common(B, Hq, Hkv, N, d, 1.0f) != FA_OK) return 0;
    if (num_splits < 1 || num_splits > FA_MAX_SPLITS) return 0;
    if (num_splits == 1) return 0;
    const size_t rows = (size_t)num_splits * B * Hq * (size_t)N;
    return round256(rows * (size_t)d * sizeof(float)) + round256(rows * sizeof(float));
}

int fa_fwd_splitkv(const void *q, const void *k, const void *v, float *o, float *lse, int B,
                   int Hq, int Hkv, int N, int d, float scale, int causal, int num_splits,
                   void *workspace, size_t workspace_bytes, void *stream)
{
    if (!q || !k || !v || !o) return FA_ERR_NULL;
    int st = check_common(B, Hq, Hkv, N, d, scale);
    if (st != FA_OK) return st;
    if (num_splits < 1 || num_splits > FA_MAX_SPLITS) return FA_ERR_SHAPE;
    // Workgroups: B * Hq * ceil(N / 256) query tiles times the chunks.
    if ((int64_t)B * Hq * ((N + 255) / 256) * num_splits > INT32_MAX) return FA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        (lse && !aligned16(lse)))
        return FA_ERR_ALIGN;
    float *opart = nullptr, *lpart = nullptr;
    if (num_splits > 1) {
        const size_t need = fa_fwd_splitkv_workspace_bytes(B, Hq, Hkv, N, d, num_splits);
        if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
        if (!aligned16(workspace)) return FA_ERR_ALIGN;
        const size_t rows = (size_t)num_splits * B * Hq * (size_t)N;
        opart = reinterpret_cast<float *>(workspace);
        lpart = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) +
                                          round256(rows * (size_t)d * sizeof(float)));
    }
    fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, scale, rescale_tau(), causal != 0,
                  exp2_poly_share(), 0, num_splits, opart, lpart,
                  reinterpret_cast<hipStream_t>(stream), nullptr, linear_map()};
    return hip_status(fa::launch_fwd(a));
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d, int deterministic)
{
    if (check_common(B, Hq, Hkv, N, d, 1.0f) != FA_OK) return 0;
    if (!valid_bwd_mode(deterministic)) return 0;
    return bwd_bytes(B, Hq, Hkv, N, d, deterministic);
}

int fa_bwd(const void *q, const void *k, const void *v, const float *o, const float *lse,
           const void *dout, float *dq, float *dk, float *dv, int B, int Hq, int Hkv, int N,
           int d, float scale, int causal, int deterministic, void *workspace,
           size_t workspace_bytes, void *stream)
{
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal, 0,
                    deterministic, workspace, workspace_bytes, stream);
}

int fa_bwd_noalloc(const void *q, const void *k, const void *v, const float *o,
                   const float *lse, const void *dout, float *dq, float *dk, float *dv, int B,
                   int Hq, int Hkv, int N, int d, float scale, int causal, int deterministic,
                   void *stream)
{
    static_assert(fa::kNoAllocScratchBytes == FA_NOALLOC_MAX_WORKSPACE, "fa.h limit");
    // Every argument check of fa_bwd first, so that nothing touches the
    // device before they pass.
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
    int st = check_common(B, Hq, Hkv, N, d, scale);
    if (st != FA_OK) return st;
    if (!valid_bwd_mode(deterministic)) return FA_ERR_SHAPE;
    const void *ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
    for (const void *p : ptrs)
        if (!aligned16(p)) return FA_ERR_ALIGN;
    if (bwd_bytes(B, Hq, Hkv, N, d, deterministic) > fa::kNoAllocScratchBytes)
        return FA_ERR_WORKSPACE;
    void *ws = nullptr;
    if (fa::noalloc_scratch(&ws) != hipSuccess) return FA_ERR_HIP;
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal, 0,
                    deterministic, ws, fa::kNoAllocScratchBytes, stream);
}

int fa_bwd_window(const void *q, const void *k, const void *v, const float *o, const float *lse,
                  const void *dout, float *dq, float *dk, float *dv, int B, int Hq, int Hkv,
                  int N, int d, float scale, int window, int deterministic, void *workspace,
                  size_t workspace_bytes, void *stream)
{
    if (window < 1) return FA_ERR_SHAPE;
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, scale, 1, window,
                    deterministic, workspace, workspace_bytes, stream);
}

#if FA_DEBUG_COUNTERS
int fa_debug_counters(unsigned long long *counters, int n)
{
    if (!counters || n < 1) return FA_ERR_NULL;
    return hip_status(fa::debug_counters(counters, n));
}

int fa_debug_atomic_tiles(float *buf, int n_slots, int tiles, int blocks, void *stream)
{
    if (!buf) return FA_ERR_NULL;
    if (n_slots < 1 || tiles < 1 || blocks < 1) return FA_ERR_SHAPE;
    if (!aligned16(buf)) return FA_ERR_ALIGN;
    return hip_status(fa::debug_atomic_tiles(buf, n_slots, tiles, blocks,
                                             reinterpret_cast<hipStream_t>(stream)));
}
#endif

int fa_fwd_alibi(const void *q, const void *k, const void *v, float *o, float *lse,
                 const float *slopes, int B, int Hq, int Hkv, int N, int d, float scale,
                 int causal, void *stream)
{
    if (!slopes) return FA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(slopes) & 3u) != 0) return FA_ERR_ALIGN;
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, 0, stream, slopes);
}

int fa_bwd_alibi(const void *q, const void *k, const void *v, const float *o, const float *lse,
                 const void *dout, float *dq, float *dk, float *dv, const float *slopes,
                 int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                 int deterministic, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!slopes) return FA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(slopes) & 3u) != 0) return FA_ERR_ALIGN;
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal, 0,
                    deterministic, workspace, workspace_bytes, stream, slopes);
}
}  // extern "C"
