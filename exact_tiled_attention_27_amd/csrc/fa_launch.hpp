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
    const float *slopes = nullptr;  // linear position bias: slope per query head, [Hq] fp32
    int linear_map = 0;             // 1: workgroups in plain order (measurement switch)
};

// How the backward sums dQ: fp32 atomics from the dK/dV kernel; a separate
// pass that owns each dQ row; the dK/dV kernel's atomics in a fixed order; or
// its atomics with pairs of key blocks sharing one set (the values of
// FA_BWD_ATOMIC .. FA_BWD_ATOMIC_PAIRED).
constexpr int kBwdAtomic = 0, kBwdSeparate = 1, kBwdOrdered = 2, kBwdAtomicPaired = 3;

// Ordered mode's int32 workspace block: the ticket counter, the count of
// timed-out waits, then (from word kSyncHead on) the turn counters, four per
// (batch, query head, 64-row tile of N rounded up to 64).
constexpr int kSyncTicket = 0, kSyncTimeouts = 1, kSyncHead = 64;
inline size_t bwd_sync_words(int BH, int N) { return kSyncHead + (size_t)BH * (((N + 63) & ~63) / 16); }

// Paired atomic mode: key blocks 2p and 2p + 1 (128 keys each) of one kv
// head form a pair; for every query tile both see, the even block hands its
// partial dQ tile to the odd one, which adds the sum, so each pair issues one
// set of dQ atomics instead of two.  Int32 block (zeroed by the preprocess):
// the header (word kSyncTimeouts counts timed-out waits), then kPairWords
// words per pair: the XCD number + 1 of each block, then per B wave the
// words of its kPairSlots ring slots (4 (e + 1) + path of the exchange e the
// slot last held) and its consumed count.  The ring itself (not zeroed)
// holds pairs x kPairSlots x 4 B waves partial tiles of 64 x d / 4 fp32.
// Longest wait of the ordered and paired modes for another workgroup: 2 s
// at the 100 MHz wall clock.
constexpr long long kWaitTicks = 200000000LL;

constexpr int kPairSlots = 4;
constexpr int kPairWords = 2 + 4 * (kPairSlots + 1);
inline size_t bwd_key_pairs(int N) { return (size_t)((N + 127) / 128 + 1) / 2; }
inline size_t bwd_pair_words(int B, int Hkv, int N)
{
    return kSyncHead + (size_t)B * Hkv * bwd_key_pairs(N) * kPairWords;
}
inline size_t bwd_pair_ring_bytes(int B, int Hkv, int N, int d)
{
    return (size_t)B * Hkv * bwd_key_pairs(N) * kPairSlots * 4 * (size_t)(64 * d);  // 64 x d / 4 fp32
}

struct BwdArgs {
    const void *q, *k, *v, *dout;
    const float *o, *lse;
    float *dq, *dk, *dv;
    float *delta;  // workspace: D_i = sum_c dO_ic O_ic, [B, Hq, N]
    float *lse2;   // workspace: LSE_i * log2(e), [B, Hq, N]
    int *sync;     // workspace: ordered mode's ticket, timeouts and turn counters, or the
                   // paired atomic mode's pair block (null in the other two modes)
    int B, Hq, Hkv, N, d;
    float scale;
    bool causal;
    int mode;      // kBwdAtomic, kBwdSeparate, kBwdOrdered or kBwdAtomicPaired
    int window;    // causal sliding window in keys (0: none)
    hipStream_t stream;
    const float *slopes = nullptr;  // linear position bias: slope per query head, [Hq] fp32
    int linear_map = 0;             // 1: workgroups in plain order (measurement switch)
    float *xring = nullptr;         // paired atomic mode: the partial-tile ring
    int pair_slots = 0;             // kPairSlots in the paired atomic mode, else 0
    int pair_memory = 0;            // 1: paired hand-over through memory even within one XCD
    long long wait_ticks = kWaitTicks;  // longest inter-workgroup wait (ordered, paired modes)
};

hipError_t launch_fwd(const FwdArgs &a);

#ifndef FA_DEBUG_COUNTERS
#define FA_DEBUG_COUNTERS 0
#endif
// Debug build (FA_DEBUG_COUNTERS=1) event counters of the forward kernels.
enum {
    kDbgRowDecisions = 0,  // rescale decisions: (row, tile) pairs after the row's first valid tile
    kDbgRowRescales,       // ... of which moved the row's reference maximum
    kDbgWaveRescales,      // waves that took the rescale branch for such a row
    kDbgTiles,             // key tiles walked, summed over workgroups
    kDbgMaskedTiles,       // ... of which took the masked path
    kDbgWorkgroups,        // workgroups launched
    kDbgCount
};
#if FA_DEBUG_COUNTERS
// Copies min(n, kDbgCount) counters to host memory, then clears them.
hipError_t debug_counters(unsigned long long *host, int n);
// The dQ atomic pattern alone (d = 128): blocks workgroups x tiles tiles of
// 64 x 128 fp32 atomic adds of 1.0 into n_slots tiles of buf.
hipError_t debug_atomic_tiles(float *buf, int n_slots, int tiles, int blocks, hipStream_t stream);
#endif
hipError_t launch_bwd(const BwdArgs &a);

// fa_bwd_noalloc's workspace: a static device array of this many bytes per
// device (FA_NOALLOC_MAX_WORKSPACE in fa.h); devices 0 .. kMaxDevices - 1.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
// Device address of the current device's array (looked up on its first use).
hipError_t noalloc_scratch(void **ptr);

// Rescale threshold: log2(256) = 8 (conditional rescaling).
constexpr float kRescaleTau = 8.0f;

// Window value the kernels receive when there is none: wider than any
// sequence, and small enough that q0 + 256 - kNoWindow cannot overflow.
constexpr int kNoWindow = 1 << 30;

}  // namespace fa
