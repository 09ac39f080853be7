// fa_bwd.hip -- backward exact attention for gfx950 (MI355X).
//
// Gradients of O = softmax(Q K^T * scale) V (the pages give no backward
// formulas; these are the analytic ones).  With P recomputed from the
// forward's log-sum-exp, P_ij = exp(scale * q_i . k_j - LSE_i):
//   dV_j = sum_i P_ij dO_i            dP_ij = dO_i . v_j
//   D_i  = sum_c dO_ic O_ic           dS_ij = P_ij (dP_ij - D_i)
//   dK_j = scale * sum_i dS_ij q_i    dQ_i  = scale * sum_j dS_ij k_j
// dQ is summed with fp32 global atomic adds, or in a separate pass that owns
// each dQ row (reproducible): the trade the FlashAttention-4 summary page
// describes under Limitations (deterministic backward) and Key Contributions
// item 3 (fewer dQ atomics).
//
// Kernels (all on the caller's stream, in order):
//   1. bwd_pre:   D_i and LSE_i * log2(e) per row into a workspace padded to
//                 64 rows per head (padding rows: D = 0, LSE2 = +inf, so
//                 P = 0); zero dQ in atomic mode.
//   2. bwd_dkdv_split: one workgroup of 8 waves per (batch, kv head, 128
//                 keys) walks 64-query tiles of every query head of the
//                 group; per 32-key slice, wave A computes S, P and dV^T,
//                 wave B dP, dS and dK^T, accumulators in registers.  Q and
//                 dO tiles arrive in LDS double-buffered; row reads feed S
//                 and dP, transposing reads feed dV^T += dO^T P and
//                 dK^T += Q^T dS, and P, dS stay in registers as B operands.
//                 Atomic mode: wave B also leaves dS^T in LDS, and at the
//                 start of the next step the B waves add dS K into dQ with
//                 fp32 atomics (the end-of-step wait finds them finished).
//   3. bwd_dq:    (deterministic mode) one workgroup per (batch, query head,
//                 128 queries) walks the key tiles, recomputes S^T, P^T,
//                 dP^T = V dO^T, dS^T, and accumulates dQ^T += K^T dS^T in
//                 registers; one plain store per element.
// Tile copies are buffer copies into LDS issued as inline assembly (so the
// compiler never drains them before unrelated LDS reads) into per-slot LDS
// arrays; each kernel settles its own global loads before the first copy and
// waits for the copies at its step barriers.
#include <mutex>
#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"
#include "fa_tiles.hpp"

#ifndef FA_DKDV_DEFER
#define FA_DKDV_DEFER 1  // deterministic mode: wave B's dK products run one step late
#endif

#ifndef FA_DQ_MIN_WAVES
#define FA_DQ_MIN_WAVES 2   // waves per SIMD the deterministic dQ kernel's registers must allow
#endif

namespace fa {

// Rows per head in the backward workspace (D, LSE2): N rounded up to 64.
__host__ __device__ inline int pad_rows(int N) { return (N + 63) & ~63; }

// ---------------------------------------------------------------- preprocess
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t *__restrict__ dout,
                                                      const float *__restrict__ o,
                                                      const float *__restrict__ lse,
                                                      float *__restrict__ delta,
                                                      float *__restrict__ lse2,
                                                      float *__restrict__ dq, int BH, int N,
                                                      int zero_dq, int *__restrict__ sync,
                                                      size_t n_sync)
{
    // Ordered mode's ticket, timeout and turn counters, or the atomic mode's
    // pair block: cleared with a grid-stride loop.
    const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (sync)
        for (size_t i = gid; i < n_sync; i += (size_t)gridDim.x * 256) sync[i] = 0;
    constexpr int TPR = D / 8;  // threads per row, 8 elements each
    const int NP = pad_rows(N);
    const size_t prow = (size_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;  // padded row
    const int part = threadIdx.x % TPR;
    const bool in_range = prow < (size_t)BH * NP;
    const int i = (int)(prow % NP);
    const size_t row = (prow / NP) * N + i;  // row of the [B, Hq, N] tensors
    const bool live = in_range && i < N;
    float acc = 0.f;
    if (live) {
        const size_t base = row * D + part * 8;
        const u32x4 raw = *reinterpret_cast<const u32x4 *>(dout + base);
        const f32x4 o0 = *reinterpret_cast<const f32x4 *>(o + base);
        const f32x4 o1 = *reinterpret_cast<const f32x4 *>(o + base + 4);
        float dv[8];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            dv[2 * j] = __builtin_bit_cast(float, raw[j] << 16);
            dv[2 * j + 1] = __builtin_bit_cast(float, raw[j] & 0xffff0000u);
        }
        acc = dv[0] * o0[0] + dv[1] * o0[1] + dv[2] * o0[2] + dv[3] * o0[3] + dv[4] * o1[0] +
              dv[5] * o1[1] + dv[6] * o1[2] + dv[7] * o1[3];
        if (zero_dq) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<f32x4 *>(dq + base) = z;
            *reinterpret_cast<f32x4 *>(dq + base + 4) = z;
        }
    }
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) acc += __shfl_xor(acc, m, 64);
    if (in_range && part == 0) {
        delta[prow] = live ? acc : 0.f;
        lse2[prow] = live ? lse[row] * kLog2e : INFINITY;
    }
}

// ------------------------------------------- dK/dV kernel, two waves per key slice
// One workgroup of 8 waves per (batch, kv head, 128 keys); the 32 keys of
// slice p are shared by two waves (both on the same SIMD):
//   wave A (w = p):     S = Q K^T, P = exp2(S * c - LSE2), dV^T += dO^T P;
//   wave B (w = p + 4): dP = dO V^T, then (after A publishes P through LDS)
//                       dS = P (dP - D), dK^T += Q^T dS.
// Each wave holds one operand set and one accumulator set (about 200
// registers), so two waves fit per SIMD and the MFMA phases of one overlap
// the exponent / elementwise phases of the other.  The Q, dO and row stages
// live in separate LDS arrays per slot (step st uses slot st % 2), so reads of
// one slot never wait for the copies into the other.
// DQ selects what the kernel does for dQ: kDqNone (the deterministic mode's
// separate pass computes it), kDqAtomic, kDqOrdered or kDqPaired.  The atomic
// modes add dQ += dS K: wave B stores dS^T to LDS after the products of step st, and the
// four B waves add that step's dQ tiles with fp32 atomics at the start of step
// st + 1 (before the mid-step barrier, after which dS^T is overwritten).
// kDqOrdered makes the adds into each 64-row dQ tile happen in ascending
// key-block order, so the fp32 sums, and dQ's bits, are the same on every run:
//   - Each workgroup draws a ticket from a counter at its start and takes
//     the work item of that ticket (key block major).  A workgroup only ever
//     waits for a smaller ticket, i.e. for a workgroup that has already
//     started, so the waits cannot deadlock whatever order the hardware
//     dispatches workgroups in.
//   - Per (query head, 64-row tile, B wave) a turn counter in the workspace
//     counts the key blocks that have added; key block kt adds when the
//     counter equals its rank among the tile's key blocks, and raises it one
//     step later, once the end-of-step wait has seen its atomics complete.
//   - Every wait is bounded (wait_ticks of the 100 MHz wall clock, 2 s by
//     default).  A wait
//     that times out is counted in the workspace, makes every later wait of
//     the launch give up at once, and the adds still happen: dQ is then the
//     correct sum in an unspecified order, and the kernel always finishes.
template <int D>
struct DkdvSplitShape {
    static constexpr int BN = 128;   // keys per workgroup (32 per wave pair)
    static constexpr int BM = 64;    // queries per step
    static constexpr int THREADS = 512;
    static constexpr int KSTEPS = D / 16;
    static constexpr int DBLK = D / 32;
    using QTile = DmaTile<BM, D, THREADS>;
    static constexpr int TILE = BM * D * 2;
    static constexpr int ROWS_BYTES = 2 * BM * 4;          // LSE2[BM], then D[BM] (fp32)
    static constexpr int X_SLICE = 64 * 32 * 4;            // P exchange per slice: 64 lanes x 32 fp32
};

constexpr int kDqNone = 0, kDqAtomic = 1, kDqOrdered = 2, kDqPaired = 3;

// Waits (the whole wave) until *turn == want, bounded as described above
// (ticks: the longest wait, in 100 MHz wall-clock ticks).
__device__ __forceinline__ void wait_turn(const int *turn, int want, int *sync, int lane,
                                          long long ticks)
{
    int seen = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(turn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (seen != want) {
        const long long t0 = wall_clock64();
        while (true) {
            __builtin_amdgcn_s_sleep(2);
            seen = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(turn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            if (seen == want) break;
            if (__builtin_amdgcn_readfirstlane(__hip_atomic_load(
                    sync + kSyncTimeouts, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0)
                break;
            if (wall_clock64() - t0 > ticks) {
                if (lane == 0)
                    __hip_atomic_fetch_add(sync + kSyncTimeouts, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    // The dQ adds that follow are issued only once the counter load has
    // returned (the branch above needs its value); keep the compiler from
    // moving them above the wait.
    asm volatile("" ::: "memory");
}

// Cache-policy bits of a buffer load or store: sc1, device scope (the
// access is coherent for every XCD of the device).
constexpr int kSc1 = 16;

// Number of the XCD (accelerator complex die) this wave runs on: the
// hardware register XCC_ID, bits 3:0.
__device__ __forceinline__ int xcd_id()
{
    return __builtin_amdgcn_s_getreg((31 << 11) | 20) & 15;  // hwreg(HW_REG_XCC_ID)
}

// BIAS: the linear position bias, slopes[hq] * (key - query), enters P's
// recomputation (added to the raw score as slope / scale * (key - query)).
template <int D, bool CAUSAL, int DQ, bool BIAS = false>
__global__ __launch_bounds__(512) void bwd_dkdv_split_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ dout,
    const float *__restrict__ lse2, const float *__restrict__ delta, float *__restrict__ dq,
    float *__restrict__ dk, float *__restrict__ dv, int Hq, int Hkv, int N, int BHkv, int KT,
    float scale, float scale_log2, int window, int *__restrict__ sync,
    const float *__restrict__ slopes, int linear_map, float *__restrict__ xring, int pair_slots,
    int pair_memory, long long wait_ticks)
{
    using S = DkdvSplitShape<D>;
    constexpr bool ATOMIC_DQ = DQ != kDqNone;
    constexpr bool ORDERED = DQ == kDqOrdered;
    // Deterministic mode: wave B's dK^T += Q^T dS of step st runs at the start
    // of step st + 1, beside wave A's score products and exponentials, where
    // B would otherwise wait at the mid-step barrier with the matrix core idle.
    // Q tile st must then outlive step st, so the stages rotate over three
    // slots (the atomic modes keep two: their K and dS^T arrays leave no room).
    constexpr bool DEFER = !ATOMIC_DQ && FA_DKDV_DEFER;
    constexpr int NSLOT = DEFER ? 3 : 2;
    // Atomic mode only: the workgroup's K rows (B operand of dQ = dS K) and
    // the step's dS^T [BN keys][BM queries] (A operand, transposing reads).
    __shared__ __attribute__((aligned(16))) char k_lds[ATOMIC_DQ ? S::BN * D * 2 : 16];
    __shared__ __attribute__((aligned(16))) char dst_lds[ATOMIC_DQ ? S::BN * S::BM * 2 : 16];
    __shared__ __attribute__((aligned(16))) char q_lds0[S::TILE];
    __shared__ __attribute__((aligned(16))) char q_lds1[S::TILE];
    __shared__ __attribute__((aligned(16))) char do_lds0[S::TILE];
    __shared__ __attribute__((aligned(16))) char do_lds1[S::TILE];
    __shared__ __attribute__((aligned(16))) char rows0[S::ROWS_BYTES];
    __shared__ __attribute__((aligned(16))) char rows1[S::ROWS_BYTES];
    __shared__ __attribute__((aligned(16))) char q_lds2[DEFER ? S::TILE : 16];
    __shared__ __attribute__((aligned(16))) char do_lds2[DEFER ? S::TILE : 16];
    __shared__ __attribute__((aligned(16))) char rows2[DEFER ? S::ROWS_BYTES : 16];
    __shared__ __attribute__((aligned(16))) char xchg_lds[4 * S::X_SLICE];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slice = wave & 3;
    const bool wave_a = wave < 4;
    const int h = lane >> 5, col = lane & 31;
    const int g16 = lane >> 4;

    int bg, kt;
    if (ORDERED) {
        __shared__ int ticket;
        if (tid == 0)
            ticket = __hip_atomic_fetch_add(sync + kSyncTicket, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int hw = __builtin_amdgcn_readfirstlane(ticket);
        if (hw >= BHkv * KT) {  // counter not cleared by the preprocess: give up
            if (tid == 0)
                __hip_atomic_fetch_add(sync + kSyncTimeouts, 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        kt = hw / BHkv;
        bg = hw % BHkv;
    } else if (DQ == kDqPaired && pair_slots > 0) {
        // Workgroups hw and hw + 8 (same hw % 8, so the same XCD under the
        // round-robin dispatch) are the two key blocks of one pair:
        // hw = 16 a + 8 m + x gives pair 8 a + x, member m.  With B Hkv a
        // multiple of 8 each XCD works through whole heads (their Q and dO
        // stay in its L2).  The grid is rounded up to 16: ids past the last
        // pair, and the missing partner of an odd block count, exit here.
        const int P = (KT + 1) / 2;
        const int hw = blockIdx.x;
        const int pid = (hw >> 4) * 8 + (hw & 7), m = (hw >> 3) & 1;
        if (pid >= BHkv * P) return;
        int p;
        if (!linear_map && BHkv % kNumXcd == 0) {
            const int per = BHkv / kNumXcd, a = pid / kNumXcd, x = pid % kNumXcd;
            bg = x * per + a / P;
            p = a % P;
        } else {
            bg = pid / P;
            p = pid % P;
        }
        kt = 2 * p + m;
        if (kt >= KT) return;
    } else {
        xcd_tile_map(blockIdx.x, BHkv, KT, false, linear_map, bg, kt);
    }
    const int b = bg / Hkv, g = bg % Hkv;
    const int grp = Hq / Hkv;
    const int NP = pad_rows(N);
    const int kv0 = kt * S::BN;
    const int key = kv0 + slice * 32 + col;  // the key this lane owns in S / dP / dS

    // Wave A keeps K rows (B operand of S), wave B keeps V rows (of dP).
    const uint16_t *kvh = (wave_a ? k : v) + ((size_t)b * Hkv + g) * N * D;
    bf16x8 kvf[S::KSTEPS];
#pragma unroll
    for (int s = 0; s < S::KSTEPS; s++)
        kvf[s] = __builtin_bit_cast(bf16x8, gload16(kvh, ((size_t)key * D + 16 * s + 8 * h) * 2, key < N));

    f32x16 acc[S::DBLK];  // A: dV^T, B: dK^T
#pragma unroll
    for (int db = 0; db < S::DBLK; db++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[db][r] = 0.f;

    uint32_t rowoff[S::KSTEPS];
#pragma unroll
    for (int s = 0; s < S::KSTEPS; s++) rowoff[s] = tile_off(col, 2 * s + h, D);
    uint32_t troff[S::DBLK][2];
#pragma unroll
    for (int db = 0; db < S::DBLK; db++)
#pragma unroll
        for (int rho = 0; rho < 2; rho++)
            troff[db][rho] = tr_off(8 * rho + 4 * h, 32 * db + 16 * (g16 & 1), lane, D);
    char *xchg = xchg_lds + slice * S::X_SLICE + lane * 16;  // + (qb*4 + gq) * 1024

    // Query tiles that see the workgroup's keys: from the diagonal on
    // (causal), up to key kv0 + BN - 1 + window - 1 (sliding window).
    const int first_qt = CAUSAL ? kv0 / S::BM : 0;
    const int n_qt_all = (N + S::BM - 1) / S::BM;
    const int n_qt = CAUSAL ? min(n_qt_all, (kv0 + S::BN + window - 2) / S::BM + 1) : n_qt_all;
    const int steps_per_head = n_qt - first_qt;
    const int n_steps = grp * steps_per_head;
    // Atomic mode with a pair block (pair_slots > 0): key blocks 2p and
    // 2p + 1 walk the query tiles both of them see, [c_lo, c_hi) of every
    // query head, first and in the same order (exchange e = step e), then
    // each its own remaining tiles.  Otherwise c_lo = c_hi = first_qt and
    // the walk is head-major in tile order.
    int c_lo = first_qt, c_hi = first_qt;
    const bool paired = DQ == kDqPaired && pair_slots > 0 && (kt ^ 1) < KT;
    if (paired) {
        const int pk = kt ^ 1;
        const int p_first = CAUSAL ? pk * S::BN / S::BM : 0;
        const int p_nqt =
            CAUSAL ? min(n_qt_all, (pk * S::BN + S::BN + window - 2) / S::BM + 1) : n_qt_all;
        c_lo = max(first_qt, p_first);
        c_hi = min(n_qt, p_nqt);
        if (c_hi <= c_lo) c_lo = c_hi = first_qt;
    }
    const int n_common = grp * (c_hi - c_lo);
    const int n_extra = steps_per_head - (c_hi - c_lo);  // per head
    // Local query head and 64-row tile of step st.
    auto tile_of = [&](int st, int &hl, int &qt) {
        if constexpr (DQ != kDqPaired) {
            hl = st / steps_per_head;
            qt = first_qt + st % steps_per_head;
            return;
        }
        if (st < n_common) {
            hl = st / (c_hi - c_lo);
            qt = c_lo + st % (c_hi - c_lo);
        } else {
            const int e = st - n_common;
            hl = e / n_extra;
            const int j = e % n_extra;
            qt = j < c_lo - first_qt ? first_qt + j : c_hi + (j - (c_lo - first_qt));
        }
        // Uniform per wave: keep them in scalar registers (tile copy bases).
        hl = __builtin_amdgcn_readfirstlane(hl);
        qt = __builtin_amdgcn_readfirstlane(qt);
    };

    typename S::QTile qtile;
    qtile.init(wave, lane);
    // Step st's tiles: Q and dO rows qs .. qs + 63 of query head hq, and the
    // tile's LSE2 and D rows (padded workspace, always in range): wave 0's
    // lanes 0-15 fetch LSE2, lanes 16-31 fetch D, 16 bytes each.
    auto issue = [&](int st, auto slot) {
        constexpr int P = decltype(slot)::value;
        int hl, qt;
        tile_of(st, hl, qt);
        const int hq = g * grp + hl;
        const int qs = qt * S::BM;
        const size_t ho = ((size_t)b * Hq + hq) * N;
        qtile.issue(make_rsrc(q + ho * D, (uint32_t)N * D * 2), qs, N,
                    P == 0 ? q_lds0 : P == 1 ? q_lds1 : q_lds2, wave);
        qtile.issue(make_rsrc(dout + ho * D, (uint32_t)N * D * 2), qs, N,
                    P == 0 ? do_lds0 : P == 1 ? do_lds1 : do_lds2, wave);
        if (wave == 0) {
            const size_t hrow = ((size_t)b * Hq + hq) * NP;
            lds_void_t *dst = (lds_void_t *)(P == 0 ? rows0 : P == 1 ? rows1 : rows2);
            if (lane < 16)
                lds_dma16_buf(make_rsrc(lse2 + hrow, (uint32_t)NP * 4), 16 * lane, qs * 4, dst);
            else if (lane < 32)
                lds_dma16_buf(make_rsrc(delta + hrow, (uint32_t)NP * 4), 16 * (lane - 16), qs * 4, dst);
        }
    };

    // Atomic mode, B waves: dQ[BM x D] += dS[BM x BN] K[BN x D] for step st,
    // whose dS^T the B waves left in dst_lds; the 2 * DBLK tiles of 32 x 32
    // are spread over the four B waves, each tile added with fp32 atomics
    // (lanes 0-31 and 32-63 cover 128 contiguous bytes of a dQ row each).
    // Ordered mode: this B wave's turn counter for step st's dQ tile, and the
    // rank of key block kt among the key blocks that add into that tile
    // (those whose query range, first_qt .. n_qt - 1 above, holds it).
    auto turn_of = [&](int st) {
        int hl, qt;
        tile_of(st, hl, qt);
        const int hq = g * grp + hl;
        return sync + kSyncHead + (((size_t)b * Hq + hq) * (NP / S::BM) + qt) * 4 + slice;
    };
    auto rank_of = [&](int st) {
        int hl, qt;
        tile_of(st, hl, qt);
        const int num = S::BM * qt - (S::BN - 2) - window;
        return kt - (CAUSAL && num > 0 ? (num + S::BN - 1) / S::BN : 0);
    };
    // The dQ adds and the turn counters are device-scope atomics, performed
    // at the device's coherence point, not in an XCD's L2: once the wave's
    // adds have completed (vmcnt(0)), raising the counter orders them before
    // every add issued after a wave has seen the raised value.  No L2
    // write-back or invalidate is needed for that (an agent-scope
    // release/acquire fence pair, which does both, made this mode five times
    // slower).
    auto release = [&](int st) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (lane == 0) __hip_atomic_fetch_add(turn_of(st), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // dQ tile tt (32 x 32) of the step whose dS^T is in dst_lds, unscaled.
    auto dq_tile = [&](int tt) {
        const int qb = tt / S::DBLK, db = tt % S::DBLK;
        const uint32_t a0 = tr_off(8 * h, 32 * qb + 16 * (g16 & 1), lane, S::BM);
        const uint32_t a1 = tr_off(8 * h + 4, 32 * qb + 16 * (g16 & 1), lane, S::BM);
        const uint32_t b0 = tr_off(8 * h, 32 * db + 16 * (g16 & 1), lane, D);
        const uint32_t b1 = tr_off(8 * h + 4, 32 * db + 16 * (g16 & 1), lane, D);
        f32x16 c = {};
#pragma unroll
        for (int ks = 0; ks < S::BN / 16; ks++) {
            const char *al = dst_lds + 16 * ks * S::BM * 2;
            const char *bl = k_lds + 16 * ks * D * 2;
            c = mfma32(join_bf16x8(lds_read_tr16(al, a0), lds_read_tr16(al, a1)),
                       join_bf16x8(lds_read_tr16(bl, b0), lds_read_tr16(bl, b1)), c);
        }
        return c;
    };
    // dQ[qs + tile tt rows] += scale * c with fp32 atomics.
    auto dq_add = [&](float *dqh, int qs, int tt, const f32x16 &c) {
        const int qb = tt / S::DBLK, db = tt % S::DBLK;
        float *dqt = dqh + (size_t)(qs + 32 * qb + 4 * h) * D + 32 * db + col;
        if (qs + S::BM <= N) {
#pragma unroll
            for (int r = 0; r < 16; r++)
                unsafeAtomicAdd(dqt + (8 * (r >> 2) + (r & 3)) * D, c[r] * scale);
        } else {
#pragma unroll
            for (int r = 0; r < 16; r++)
                if (qs + 32 * qb + 4 * h + 8 * (r >> 2) + (r & 3) < N)
                    unsafeAtomicAdd(dqt + (8 * (r >> 2) + (r & 3)) * D, c[r] * scale);
        }
    };
    constexpr int TILES = 2 * S::DBLK;  // 32 x 32 dQ tiles per step
    constexpr int NT = TILES / 4;       // ... per B wave: tiles slice, slice + 4, ...
    // Paired atomic mode, exchange e = st (a step both key blocks of the
    // pair walk) of this B wave; the partner block's wave with the same slice
    // holds the other partial of the same dQ tiles.  Fixed roles: the even
    // block (producer) hands its partial over, the odd block (consumer) adds
    // both and issues the only atomics.
    //  - The producer waits until ring slot e % R is free (the consumer's
    //    count of consumed exchanges >= e - R + 1), stores its partial there,
    //    waits for the stores, then writes 4 (e + 1) + path into the slot's
    //    word.  path 0: plain stores, which land in the L2 of its XCD (taken
    //    when the consumer has published the same XCD number, unless
    //    pair_memory asks for path 1 throughout); path 1: device-scope (sc1)
    //    stores, visible from any XCD.
    //  - The consumer waits for that word, loads the partial (after an L1
    //    invalidate, or with device-scope loads), adds it, issues the
    //    atomics for both blocks and raises its consumed count.
    //  - Both waits are bounded (wait_ticks, counted in word kSyncTimeouts;
    //    after one timeout every later wait gives up at once, so the kernel
    //    always finishes).  A timeout leaves dq incomplete, and the count
    //    tells the caller so.  The producer never waits for anything the
    //    consumer needs from it, and the consumer only for the producer's
    //    earlier exchanges, so no order of dispatch can deadlock them.
    const size_t pair_id = (size_t)bg * ((KT + 1) / 2) + (kt >> 1);
    int *const pwords = sync + kSyncHead + pair_id * kPairWords;  // this pair's words
    int *const slot_words = pwords + 2 + slice * (kPairSlots + 1);  // R slot words, consumed count
    int *const consumed = slot_words + kPairSlots;
    const bool producer = (kt & 1) == 0;
    const int my_xcd = xcd_id() + 1;
    if (DQ == kDqPaired && paired && tid == 0)
        __hip_atomic_store(pwords + (kt & 1), my_xcd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int partner_xcd = 0;  // producer: the consumer's published XCD number, once known
    // Bounded wait (the whole wave) until *w >= want; returns the last value.
    auto wait_at_least = [&](const int *w, int want, int seen) {
        if (seen >= want) return seen;
        const long long t0 = wall_clock64();
        while (true) {
            seen = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            if (seen >= want) break;
            if (__builtin_amdgcn_readfirstlane(__hip_atomic_load(
                    sync + kSyncTimeouts, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0)
                break;
            if (wall_clock64() - t0 > wait_ticks) {
                if (lane == 0)
                    __hip_atomic_fetch_add(sync + kSyncTimeouts, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        // The slot accesses that follow depend on this value (branch).
        asm volatile("" ::: "memory");
        return seen;
    };
    // Read ahead at the end of step st, once dS is known, so that the value
    // is back when the exchange runs at the start of step st + 1: the
    // producer reads the consumed count, the consumer the slot word.
    int pre_seen = 0;
    auto arrive = [&](int st) {
        const int *w = producer ? consumed : slot_words + st % kPairSlots;
        if (lane == 0) pre_seen = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto ring_rsrc = [&](int st) {
        return __builtin_amdgcn_make_buffer_rsrc(
            xring + ((pair_id * kPairSlots + st % kPairSlots) * 4 + slice) * (16 * D), 0, 16 * D * 4,
            0x00020000);
    };
    // Producer: hand over c (returns false when a wait timed out: then c
    // was not handed over and the caller adds it itself).
    auto hand_over = [&](int st, const f32x16 (&c)[NT]) __attribute__((always_inline)) {
        int seen = wait_at_least(consumed, st - kPairSlots + 1,
                                 __builtin_amdgcn_readfirstlane(pre_seen));
        if (seen < st - kPairSlots + 1) return false;
        if (partner_xcd == 0)
            partner_xcd = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(pwords + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        const bool l2 = partner_xcd == my_xcd && !pair_memory;
        const auto rs = ring_rsrc(st);
#pragma unroll
        for (int i = 0; i < NT; i++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const f32x4 v4 = {c[i][4 * j], c[i][4 * j + 1], c[i][4 * j + 2], c[i][4 * j + 3]};
                const u32x4 u = __builtin_bit_cast(u32x4, v4);
                const int off = ((i * 4 + j) * 64 + lane) * 16;
                if (l2)
                    __builtin_amdgcn_raw_buffer_store_b128(u, rs, off, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b128(u, rs, off, 0, kSc1);
            }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (lane == 0)
            __hip_atomic_store(slot_words + st % kPairSlots, 4 * (st + 1) + (l2 ? 0 : 1),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return true;
    };
    // Consumer: load the producer's partial into p (zeros when the wait
    // timed out: then only this block's own partial is added).
    auto take_over = [&](int st, f32x16 (&p)[NT]) __attribute__((always_inline)) {
        const int v = wait_at_least(slot_words + st % kPairSlots, 4 * (st + 1),
                                    __builtin_amdgcn_readfirstlane(pre_seen));
        const bool ok = v >= 4 * (st + 1);
        const bool l2 = (v & 3) == 0;
        const auto rs = ring_rsrc(st);
        // Plain path: the partner ran on this XCD and its stores are in this
        // L2; drop any copy of the slot this compute unit's L1 holds from an
        // earlier exchange.
        if (ok && l2) asm volatile("buffer_inv sc0" ::: "memory");
#pragma unroll
        for (int i = 0; i < NT; i++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int off = ((i * 4 + j) * 64 + lane) * 16;
                f32x4 v4 = {0.f, 0.f, 0.f, 0.f};
                if (ok)
                    v4 = __builtin_bit_cast(
                        f32x4, l2 ? __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0)
                                  : __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kSc1));
#pragma unroll
                for (int r = 0; r < 4; r++) p[i][4 * j + r] = v4[r];
            }
    };
    auto dq_update = [&](int st) __attribute__((always_inline)) {
        int hl, qt;
        tile_of(st, hl, qt);
        const int hq = g * grp + hl;
        const int qs = qt * S::BM;
        float *dqh = dq + ((size_t)b * Hq + hq) * N * D;
        if (DQ == kDqPaired && paired && st < n_common) {
            f32x16 c[NT];
            if (!producer) {
                // Consumer: issue the partial's loads before this block's
                // own dQ products, so their latency hides behind the matrix
                // work.
                f32x16 pl[NT];
                take_over(st, pl);
#pragma unroll
                for (int i = 0; i < NT; i++) c[i] = dq_tile(slice + 4 * i) + pl[i];
#pragma unroll
                for (int i = 0; i < NT; i++) dq_add(dqh, qs, slice + 4 * i, c[i]);
                // The slot's loads have returned (the sums used them): free
                // it, after those uses in program order.
                asm volatile("" ::: "memory");
                if (lane == 0)
                    __hip_atomic_store(consumed, st + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return;
            }
            // Producer.
#pragma unroll
            for (int i = 0; i < NT; i++) c[i] = dq_tile(slice + 4 * i);
            if (!hand_over(st, c)) {
#pragma unroll
                for (int i = 0; i < NT; i++) dq_add(dqh, qs, slice + 4 * i, c[i]);
            }
            return;
        }
#pragma unroll
        for (int tt = slice; tt < TILES; tt += 4) {
            const f32x16 c = dq_tile(tt);
            if (ORDERED && tt == slice) wait_turn(turn_of(st), rank_of(st), sync, lane, wait_ticks);
            dq_add(dqh, qs, tt, c);
        }
    };

    // A: dV^T += dO^T P.  B: dK^T += Q^T dS.  tl: the dO (A) or Q (B) tile,
    // read transposed; bo: P or dS as B operands.
    auto tr_products = [&](const char *tl, const bf16x8(&bo)[4]) {
#pragma unroll
        for (int ks = 0; ks < 4; ks++)
#pragma unroll
            for (int db = 0; db < S::DBLK; db++) {
                const uint32_t o0 = troff[db][0] + 16 * ks * D * 2;
                const uint32_t o1 = troff[db][1] + 16 * ks * D * 2;
                acc[db] = mfma32(join_bf16x8(lds_read_tr16(tl, o0), lds_read_tr16(tl, o1)), bo[ks], acc[db]);
            }
    };
    bf16x8 bprev[4];  // deferred mode, B waves: the previous step's dS
#pragma unroll
    for (int i = 0; i < 4; i++) bprev[i] = bf16x8{};

    auto step = [&](auto slot, int st) {
        constexpr int P = decltype(slot)::value;
        int hl_st, qt_st;
        tile_of(st, hl_st, qt_st);
        const int qs = qt_st * S::BM;
        constexpr int PN = (P + 1) % NSLOT;          // slot of step st + 1
        constexpr int PP = (P + NSLOT - 1) % NSLOT;  // slot of step st - 1
        const char *ql = P == 0 ? q_lds0 : P == 1 ? q_lds1 : q_lds2;
        const char *dol = P == 0 ? do_lds0 : P == 1 ? do_lds1 : do_lds2;
        const char *rows = P == 0 ? rows0 : P == 1 ? rows1 : rows2;
        // This lane's byte offset into the row stage (its rows are 4 h + 8 j
        // + ...); laundered each step so that the compiler does not keep one
        // hoisted offset register per row group, which costs spills.
        uint32_t hoff = 16 * h;
        asm volatile("" : "+v"(hoff));
        // Ordered mode: step st - 2's adds completed at the last end-of-step
        // wait; publish them before this step's copies are in flight (the
        // release waits for every outstanding memory operation of the wave).
        if (ORDERED && !wave_a && st > 1) release(st - 2);
        // Paired atomic mode: the B waves add (or hand over) the previous
        // step's dQ before this step's copies are in flight, so that a first
        // arrival's wait for its ring stores waits for nothing else.
        if (paired && !wave_a && st > 0) dq_update(st - 1);
        if (st + 1 < n_steps) issue(st + 1, std::integral_constant<int, PN>{});
        // Deferred mode, B waves: dK^T += Q^T dS of step st - 1 (its Q tile
        // is still in slot PP, its dS in bprev) while the A waves compute S.
        if (DEFER && !wave_a && st > 0) tr_products(PP == 0 ? q_lds0 : PP == 1 ? q_lds1 : q_lds2, bprev);
        // Atomic modes: the B waves add the previous step's dS K into dQ first
        // (no score registers live yet), while the A waves start on S.
        if (ATOMIC_DQ && !paired && !wave_a && st > 0) dq_update(st - 1);

        // A: S = Q K^T.  B: dP = dO V^T.  (rows = queries, one key per lane)
        const char *rl = wave_a ? ql : dol;
        f32x16 x[2];
        // Operands read two k-steps ahead of the products that use them.
        bf16x8 ra[S::KSTEPS][2];
#pragma unroll
        for (int s = 0; s < 2; s++)
#pragma unroll
            for (int qb = 0; qb < 2; qb++) ra[s][qb] = lds_read_bf16x8(rl, rowoff[s] + qb * 32 * D * 2);
#pragma unroll
        for (int s = 0; s < S::KSTEPS; s++) {
            if (s + 2 < S::KSTEPS) {
#pragma unroll
                for (int qb = 0; qb < 2; qb++)
                    ra[s + 2][qb] = lds_read_bf16x8(rl, rowoff[s + 2] + qb * 32 * D * 2);
            }
#pragma unroll
            for (int qb = 0; qb < 2; qb++) {
                x[qb] = mfma32(ra[s][qb], kvf[s], s == 0 ? f32x16{} : x[qb]);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // then one product
            }
        }

        if (wave_a) {
            // P = exp2(s * c - LSE2); masked pairs get a -inf exponent.
            const bool need_mask = kv0 + S::BN > N || qs + S::BM > N ||
                                   (CAUSAL && (qs < kv0 + S::BN - 1 || qs + S::BM - 1 - kv0 >= window));
            // Slope / scale of this step's query head.
            const float bias_a =
                BIAS ? slopes[g * grp + hl_st] * (kLog2e / scale_log2) : 0.f;
            auto softmax = [&](auto masked) {
                constexpr bool MASK = decltype(masked)::value;
#pragma unroll
                for (int qb = 0; qb < 2; qb++)
#pragma unroll
                    for (int gq = 0; gq < 4; gq++) {
                        const int qr = 32 * qb + 8 * gq + 4 * h;
                        const f32x4 l2 = lds_read_f32x4(rows, hoff + (32 * qb + 8 * gq) * 4);
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            float xs = x[qb][4 * gq + i];
                            if (BIAS) xs += bias_a * (float)(key - (qs + qr + i));
                            float e = __builtin_fmaf(xs, scale_log2, -l2[i]);
                            if (MASK) {
                                const int qi = qs + qr + i;
                                const bool dead = key >= N || qi >= N ||
                                                  (CAUSAL && (key > qi || qi - key >= window));
                                e = dead ? -INFINITY : e;
                            }
                            x[qb][4 * gq + i] = exp2_hw(e);
                        }
                        const f32x4 pv = {x[qb][4 * gq], x[qb][4 * gq + 1], x[qb][4 * gq + 2], x[qb][4 * gq + 3]};
                        *reinterpret_cast<f32x4 *>(xchg + (qb * 4 + gq) * 1024) = pv;
                    }
            };
            if (need_mask)
                softmax(std::true_type{});
            else
                softmax(std::false_type{});
        }
        lds_barrier();  // P of every slice published (and, atomic mode, dS^T consumed)

        bf16x8 bop[4];  // A: P, B: dS (B operands, key order of the accumulator rows)
        if (wave_a) {
#pragma unroll
            for (int qb = 0; qb < 2; qb++) {
                bop[2 * qb] = pack_half(x[qb], 0);
                bop[2 * qb + 1] = pack_half(x[qb], 1);
            }
        } else {
#pragma unroll
            for (int qb = 0; qb < 2; qb++) {
#pragma unroll
                for (int gq = 0; gq < 4; gq++) {
                    const f32x4 dl = lds_read_f32x4(rows, hoff + (S::BM + 32 * qb + 8 * gq) * 4);
                    const f32x4 pv = *reinterpret_cast<const f32x4 *>(xchg + (qb * 4 + gq) * 1024);
#pragma unroll
                    for (int i = 0; i < 4; i++) x[qb][4 * gq + i] = pv[i] * (x[qb][4 * gq + i] - dl[i]);
                }
                bop[2 * qb] = pack_half(x[qb], 0);
                bop[2 * qb + 1] = pack_half(x[qb], 1);
            }
            if (ATOMIC_DQ) {
                // dS^T row = this lane's key; bop[ks] holds queries
                // 16 ks + 4 h + 0..3 and 16 ks + 8 + 4 h + 0..3: the two
                // halves of chunks 2 ks and 2 ks + 1 selected by h.
                const int kin = slice * 32 + col;
#pragma unroll
                for (int ks = 0; ks < 4; ks++) {
                    const i16x8 w = __builtin_bit_cast(i16x8, bop[ks]);
                    const i16x4 lo = __builtin_shufflevector(w, w, 0, 1, 2, 3);
                    const i16x4 hi = __builtin_shufflevector(w, w, 4, 5, 6, 7);
                    *reinterpret_cast<i16x4 *>(dst_lds + tile_off(kin, 2 * ks, S::BM) + 8 * h) = lo;
                    *reinterpret_cast<i16x4 *>(dst_lds + tile_off(kin, 2 * ks + 1, S::BM) + 8 * h) = hi;
                }
                if (DQ == kDqPaired && paired && st < n_common) arrive(st);
            }
        }
        if (DEFER && !wave_a) {
#pragma unroll
            for (int i = 0; i < 4; i++) bprev[i] = bop[i];
        } else {
            tr_products(wave_a ? dol : ql, bop);
        }
        dma_barrier();  // next stage landed; this stage and the exchange are free
    };
    using Slot0 = std::integral_constant<int, 0>;
    using Slot1 = std::integral_constant<int, 1>;

    // First copies while the K/V row loads are in flight; the barrier drains
    // both, and the loads are settled before the loop's copies start.
    if (ATOMIC_DQ) {
        DmaTile<S::BN, D, S::THREADS> ktile;
        ktile.init(wave, lane);
        ktile.issue(make_rsrc(k + ((size_t)b * Hkv + g) * N * D, (uint32_t)N * D * 2), kv0, N,
                    k_lds, wave);
    }
    if (n_steps > 0) issue(0, Slot0{});
    dma_barrier();
#pragma unroll
    for (int s = 0; s < S::KSTEPS; s++) settle(kvf[s]);
    int st = 0;
    if constexpr (DEFER) {
        using Slot2 = std::integral_constant<int, 2>;
        for (; st + 3 <= n_steps; st += 3) {
            step(Slot0{}, st);
            step(Slot1{}, st + 1);
            step(Slot2{}, st + 2);
        }
        // Then the last step's dK products (its Q tile is still in its slot).
        if (st + 2 <= n_steps) {
            step(Slot0{}, st);
            step(Slot1{}, st + 1);
            if (!wave_a) tr_products(q_lds1, bprev);
        } else if (st + 1 <= n_steps) {
            step(Slot0{}, st);
            if (!wave_a) tr_products(q_lds0, bprev);
        } else if (n_steps > 0 && !wave_a) {
            tr_products(q_lds2, bprev);
        }
    } else {
        for (; st + 2 <= n_steps; st += 2) {
            step(Slot0{}, st);
            step(Slot1{}, st + 1);
        }
        if (st < n_steps) step(Slot0{}, st);
    }
    if (ATOMIC_DQ && !wave_a && n_steps > 0) {
        if (ORDERED && n_steps > 1) release(n_steps - 2);
        dq_update(n_steps - 1);
        if (ORDERED) release(n_steps - 1);
    }

    if (key < N) {
        float *out = (wave_a ? dv : dk) + (((size_t)b * Hkv + g) * N + key) * D;
        const float f = wave_a ? 1.f : scale;
#pragma unroll
        for (int db = 0; db < S::DBLK; db++)
#pragma unroll
            for (int gq = 0; gq < 4; gq++) {
                f32x4 val = {acc[db][4 * gq] * f, acc[db][4 * gq + 1] * f, acc[db][4 * gq + 2] * f,
                             acc[db][4 * gq + 3] * f};
                *reinterpret_cast<f32x4 *>(out + 32 * db + 8 * gq + 4 * h) = val;
            }
    }
}

// ------------------------------------------------- deterministic dQ kernel
template <int D>
struct DqShape {
    static constexpr int BM = 128;  // queries per workgroup (32 per wave)
    static constexpr int BN = 64;   // keys per tile
    static constexpr int THREADS = 256;
    static constexpr int KSTEPS = D / 16;
    static constexpr int DBLK = D / 32;
    using Tile = DmaTile<BN, D, THREADS>;   // K and V tiles, row-major
    static constexpr int TILE = BN * D * 2;
};

// K and V tiles live in four separate LDS arrays (slot t % 2 of each), so
// that reads of one slot never wait for the copies into the other.
// DELTA: instead of dQ, the row terms D_i = sum_j P_ij dP_ij from this
// pass's own recomputed P and dP (written to delta_out; delta and dq are
// unused).  Equal to sum_c dO_ic O_ic for the exact O; computed this way it
// is consistent with the P the other backward kernels recompute, so
// sum_j dS_ij = 0 holds to fp32 rounding even where the forward's O carries
// the rounding of its bf16 P.
template <int D, bool CAUSAL, bool BIAS = false, bool DELTA = false>
__global__ __launch_bounds__(256, FA_DQ_MIN_WAVES) void bwd_dq_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ dout,
    const float *__restrict__ lse2, const float *__restrict__ delta, float *__restrict__ dq,
    int Hq, int Hkv, int N, int BH, int QT, float scale, float scale_log2, int window,
    const float *__restrict__ slopes, float *__restrict__ delta_out, int linear_map)
{
    using S = DqShape<D>;
    __shared__ __attribute__((aligned(16))) char k_lds0[S::TILE];
    __shared__ __attribute__((aligned(16))) char k_lds1[S::TILE];
    __shared__ __attribute__((aligned(16))) char v_lds0[S::TILE];
    __shared__ __attribute__((aligned(16))) char v_lds1[S::TILE];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, col = lane & 31;
    const int g16 = lane >> 4;

    int bh, qt;
    xcd_tile_map(blockIdx.x, BH, QT, CAUSAL, linear_map, bh, qt);
    const int b = bh / Hq, hq = bh % Hq;
    const int g = hq / (Hq / Hkv);
    const int q0 = qt * S::BM;
    const int qrow = q0 + wave * 32 + col;
    const size_t head_off = ((size_t)b * Hq + hq) * N;
    const float bias_a = BIAS ? slopes[hq] * (kLog2e / scale_log2) : 0.f;  // slope / scale

    const uint16_t *qh = q + head_off * D;
    const uint16_t *doh = dout + head_off * D;
    const uint16_t *kh = k + ((size_t)b * Hkv + g) * N * D;
    const uint16_t *vh = v + ((size_t)b * Hkv + g) * N * D;

    bf16x8 qf[S::KSTEPS], df[S::KSTEPS];
#pragma unroll
    for (int s = 0; s < S::KSTEPS; s++) {
        qf[s] = __builtin_bit_cast(bf16x8, gload16(qh, ((size_t)qrow * D + 16 * s + 8 * h) * 2, qrow < N));
        df[s] = __builtin_bit_cast(bf16x8, gload16(doh, ((size_t)qrow * D + 16 * s + 8 * h) * 2, qrow < N));
    }
    const size_t prow = ((size_t)b * Hq + hq) * pad_rows(N) + qrow;  // padded workspace row
    const float l2 = qrow < N ? lse2[prow] : INFINITY;
    const float dl = (qrow < N && !DELTA) ? delta[prow] : 0.f;
    float dsum[4] = {0.f, 0.f, 0.f, 0.f};  // DELTA: this lane's part of D, four chains

    // K and V row reads (A operands of S^T and dP^T): row 32 kb + col, chunk
    // 2 s + h.  K^T by transposing reads (A operand of dQ^T): keys
    // 16 ks + 8 rho + 4 h .. +3 (the key order of the dS^T registers).
    uint32_t rowoff[S::KSTEPS];
#pragma unroll
    for (int s = 0; s < S::KSTEPS; s++) rowoff[s] = tile_off(col, 2 * s + h, D);
    uint32_t troff[S::DBLK][2];
#pragma unroll
    for (int db = 0; db < S::DBLK; db++)
#pragma unroll
        for (int rho = 0; rho < 2; rho++)
            troff[db][rho] = tr_off(8 * rho + 4 * h, 32 * db + 16 * (g16 & 1), lane, D);

    f32x16 acc[S::DBLK];
#pragma unroll
    for (int db = 0; db < S::DBLK; db++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[db][r] = 0.f;

    const int n_tiles_all = (N + S::BN - 1) / S::BN;
    const int n_tiles = CAUSAL ? min(n_tiles_all, (min(q0 + S::BM, N) + S::BN - 1) / S::BN)
                               : n_tiles_all;
    // Tiles every key of which is < N and (causal) <= q0 need no mask.
    const int n_full = CAUSAL ? min(N / S::BN, (q0 + 1) / S::BN) : N / S::BN;
    // Causal sliding window: t_lo is the first tile any row sees, w_full the
    // first one every row sees whole.
    const int t_lo = CAUSAL ? max(0, q0 - window + 1) / S::BN : 0;
    const int w_full = CAUSAL ? (max(0, q0 + S::BM - window) + S::BN - 1) / S::BN : 0;

    typename S::Tile tile;
    tile.init(wave, lane);
    const BufRsrc krs = make_rsrc(kh, (uint32_t)N * D * 2);
    const BufRsrc vrs = make_rsrc(vh, (uint32_t)N * D * 2);
    auto issue = [&](int t, auto slot) {
        constexpr int P = decltype(slot)::value;
        tile.issue(krs, t * S::BN, N, P ? k_lds1 : k_lds0, wave);
        tile.issue(vrs, t * S::BN, N, P ? v_lds1 : v_lds0, wave);
    };

    // One key tile t in slot P: S^T = K Q^T, dP^T = V dO^T, P^T, dS^T, then
    // dQ^T += K^T dS^T.  Tile t + 1 is copied into the other slot meanwhile.
    auto step = [&](auto masked, auto slot, int t) {
        constexpr bool MASK = decltype(masked)::value;
        constexpr int P = decltype(slot)::value;
        const int key0 = t * S::BN;
        if (t + 1 < n_tiles) issue(t + 1, std::integral_constant<int, 1 - P>{});
        const char *kl = P ? k_lds1 : k_lds0;
        const char *vl = P ? v_lds1 : v_lds0;
        // One 32-key block at a time: S^T and dP^T of block kb (two product
        // chains, operands read two k-steps ahead), then its P^T and dS^T.
        // Keys >= N and (causal) keys after the query get a -inf exponent.
        bf16x8 dsf[S::BN / 16];
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            f32x16 st, dpt;
            bf16x8 ka[S::KSTEPS], va[S::KSTEPS];
#pragma unroll
            for (int s = 0; s < 2; s++) {
                ka[s] = lds_read_bf16x8(kl, rowoff[s] + kb * 32 * D * 2);
                va[s] = lds_read_bf16x8(vl, rowoff[s] + kb * 32 * D * 2);
            }
#pragma unroll
            for (int s = 0; s < S::KSTEPS; s++) {
                if (s + 2 < S::KSTEPS) {
                    ka[s + 2] = lds_read_bf16x8(kl, rowoff[s + 2] + kb * 32 * D * 2);
                    va[s + 2] = lds_read_bf16x8(vl, rowoff[s + 2] + kb * 32 * D * 2);
                }
                st = mfma32(ka[s], qf[s], s == 0 ? f32x16{} : st);
                dpt = mfma32(va[s], df[s], s == 0 ? f32x16{} : dpt);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // then two products
            }
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int kk = key0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                float xs = st[r];
                if (BIAS) xs += bias_a * (float)(kk - qrow);
                float x = __builtin_fmaf(xs, scale_log2, -l2);
                if (MASK) {
                    const bool dead = kk >= N || (CAUSAL && (kk > qrow || qrow - kk >= window));
                    x = dead ? -INFINITY : x;
                }
                if (DELTA)
                    dsum[r & 3] = __builtin_fmaf(exp2_hw(x), dpt[r], dsum[r & 3]);
                else
                    dpt[r] = exp2_hw(x) * (dpt[r] - dl);
            }
            if (!DELTA) {
                dsf[2 * kb] = pack_half(dpt, 0);
                dsf[2 * kb + 1] = pack_half(dpt, 1);
            }
        }
        if constexpr (DELTA) {
            dma_barrier();  // tile t + 1 landed; slot P is free
            return;
        }
        // dQ^T += K^T dS^T (contraction over the tile's keys), transposing
        // reads two products ahead.
        constexpr int NP2 = (S::BN / 16) * S::DBLK;
        i16x4 tl[NP2][2];
#pragma unroll
        for (int i = 0; i < NP2; i++) {
            const int ks = i / S::DBLK, db = i % S::DBLK;
            tl[i][0] = lds_read_tr16(kl, troff[db][0] + 16 * ks * D * 2);
            tl[i][1] = lds_read_tr16(kl, troff[db][1] + 16 * ks * D * 2);
            if (i >= 2) {
                const int j = i - 2, ksj = j / S::DBLK, dbj = j % S::DBLK;
                acc[dbj] = mfma32(join_bf16x8(tl[j][0], tl[j][1]), dsf[ksj], acc[dbj]);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);  // two transposing reads
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // then one product
            }
        }
#pragma unroll
        for (int j = NP2 - 2; j < NP2; j++) {
            const int ksj = j / S::DBLK, dbj = j % S::DBLK;
            acc[dbj] = mfma32(join_bf16x8(tl[j][0], tl[j][1]), dsf[ksj], acc[dbj]);
        }
        dma_barrier();  // tile t + 1 landed; slot P is free
    };
    using Slot0 = std::integral_constant<int, 0>;
    using Slot1 = std::integral_constant<int, 1>;

    // First copies while the Q / dO row loads are in flight; the barrier
    // drains both, and the loads are settled before the loop's copies start.
    issue(t_lo, Slot0{});
    dma_barrier();
#pragma unroll
    for (int s = 0; s < S::KSTEPS; s++) {
        settle(qf[s]);
        settle(df[s]);
    }
    settle(l2);
    settle(dl);
    // Unrolled by two so that LDS slots are compile-time constants; unmasked
    // tiles first, then the diagonal and tail tiles.
    int t = t_lo;
    for (; t < w_full && t + 2 <= n_tiles; t += 2) {  // tiles the window cuts
        step(std::true_type{}, Slot0{}, t);
        step(std::true_type{}, Slot1{}, t + 1);
    }
    for (; t + 2 <= n_full; t += 2) {
        step(std::false_type{}, Slot0{}, t);
        step(std::false_type{}, Slot1{}, t + 1);
    }
    for (; t + 2 <= n_tiles; t += 2) {
        step(std::true_type{}, Slot0{}, t);
        step(std::true_type{}, Slot1{}, t + 1);
    }
    if (t < n_tiles) step(std::true_type{}, Slot0{}, t);

    if constexpr (DELTA) {
        const float dsum_all = halves_sum((dsum[0] + dsum[1]) + (dsum[2] + dsum[3]));
        if (qrow < N && h == 0) delta_out[prow] = dsum_all;
        return;
    }
    if (qrow < N) {
        float *dqr = dq + (head_off + qrow) * D;
#pragma unroll
        for (int db = 0; db < S::DBLK; db++)
#pragma unroll
            for (int gq = 0; gq < 4; gq++) {
                f32x4 val = {acc[db][4 * gq] * scale, acc[db][4 * gq + 1] * scale,
                             acc[db][4 * gq + 2] * scale, acc[db][4 * gq + 3] * scale};
                *reinterpret_cast<f32x4 *>(dqr + 32 * db + 8 * gq + 4 * h) = val;
            }
    }
}

// ------------------------------------------------------------------ launch
template <int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs &a)
{
    (void)hipGetLastError();  // clear an error left by an earlier, unrelated call
    const int BH = a.B * a.Hq;
    const float scale_log2 = a.scale * kLog2e;
    // Atomic mode with a pair block and ring in the workspace.
    const bool pairs = a.mode == kBwdAtomicPaired;
    {
        constexpr int RPB = 256 / (D / 8);
        const size_t rows = (size_t)BH * pad_rows(a.N);
        const unsigned grid = (unsigned)((rows + RPB - 1) / RPB);
        const size_t n_sync = a.mode == kBwdOrdered ? bwd_sync_words(BH, a.N)
                              : pairs ? bwd_pair_words(a.B, a.Hkv, a.N)
                                      : (size_t)0;
        hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3(grid), dim3(256), 0, a.stream,
                           (const uint16_t *)a.dout, a.o, a.lse, a.delta, a.lse2, a.dq, BH, a.N,
                           a.mode == kBwdSeparate ? 0 : 1, n_sync ? a.sync : nullptr, n_sync);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.slopes) {
        // Linear position bias: D_i from the recomputed P and dP (see
        // bwd_dq_kernel's DELTA), replacing the preprocess's sum_c dO_ic O_ic.
        using S = DqShape<D>;
        const int QT = (a.N + S::BM - 1) / S::BM;
        hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, true, true>), dim3(BH * QT), dim3(S::THREADS),
                           0, a.stream, (const uint16_t *)a.q, (const uint16_t *)a.k,
                           (const uint16_t *)a.v, (const uint16_t *)a.dout, a.lse2,
                           (const float *)nullptr, (float *)nullptr, a.Hq, a.Hkv, a.N, BH, QT,
                           a.scale, scale_log2, a.window > 0 ? a.window : kNoWindow, a.slopes,
                           a.delta, a.linear_map);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        using S = DkdvSplitShape<D>;
        const int KT = (a.N + S::BN - 1) / S::BN;
        const int BHkv = a.B * a.Hkv;
        auto kern = a.mode == kBwdSeparate  ? bwd_dkdv_split_kernel<D, CAUSAL, kDqNone>
                    : a.mode == kBwdOrdered ? bwd_dkdv_split_kernel<D, CAUSAL, kDqOrdered>
                    : pairs                 ? bwd_dkdv_split_kernel<D, CAUSAL, kDqPaired>
                                            : bwd_dkdv_split_kernel<D, CAUSAL, kDqAtomic>;
        if (a.slopes)
            kern = a.mode == kBwdSeparate  ? bwd_dkdv_split_kernel<D, CAUSAL, kDqNone, true>
                 : a.mode == kBwdOrdered ? bwd_dkdv_split_kernel<D, CAUSAL, kDqOrdered, true>
                 : pairs                 ? bwd_dkdv_split_kernel<D, CAUSAL, kDqPaired, true>
                                         : bwd_dkdv_split_kernel<D, CAUSAL, kDqAtomic, true>;
        // Paired atomic mode: two workgroups per key-block pair, rounded up to
        // 16 (see the kernel's pair map).
        const unsigned grid =
            pairs ? (unsigned)((2 * BHkv * ((KT + 1) / 2) + 15) / 16 * 16) : (unsigned)(BHkv * KT);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(S::THREADS), 0, a.stream,
                           (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                           (const uint16_t *)a.dout, a.lse2, a.delta, a.dq, a.dk, a.dv, a.Hq,
                           a.Hkv, a.N, BHkv, KT, a.scale, scale_log2,
                           a.window > 0 ? a.window : kNoWindow,
                           a.mode == kBwdOrdered || pairs ? a.sync : nullptr, a.slopes, a.linear_map,
                           pairs ? a.xring : nullptr, pairs ? a.pair_slots : 0,
                           pairs ? a.pair_memory : 0, a.wait_ticks);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.mode == kBwdSeparate) {
        using S = DqShape<D>;
        const int QT = (a.N + S::BM - 1) / S::BM;
        auto kern = a.slopes ? bwd_dq_kernel<D, CAUSAL, true> : bwd_dq_kernel<D, CAUSAL>;
        hipError_t e;
        hipLaunchKernelGGL(kern, dim3(BH * QT), dim3(S::THREADS), 0, a.stream,
                           (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                           (const uint16_t *)a.dout, a.lse2, a.delta, a.dq, a.Hq, a.Hkv, a.N, BH,
                           QT, a.scale, scale_log2, a.window > 0 ? a.window : kNoWindow, a.slopes,
                           (float *)nullptr, a.linear_map);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

#if FA_DEBUG_COUNTERS
// Debug build only: the dQ atomics of bwd_dkdv_split_kernel's atomic modes
// without anything else, to measure the device's rate for them.  Workgroup
// w (256 threads) adds `tiles` tiles of 64 x D fp32 values into tile slot
// (7 w + 13 i) % n_slots of buf, each wave two 32 x 32 blocks per tile with
// the B waves' lane pattern (lanes 0-31 and 32-63 on 128 contiguous bytes
// of rows 4 apart).
template <int D>
__global__ __launch_bounds__(256) void dbg_atomic_tiles_kernel(float *buf, int n_slots, int tiles)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int h = lane >> 5, col = lane & 31;
    constexpr int DBLK = D / 32;
    for (int i = 0; i < tiles; i++) {
        const int slot = (int)(((long long)blockIdx.x * 7 + (long long)i * 13) % n_slots);
        float *tile = buf + (size_t)slot * 64 * D;
        for (int tt = wave; tt < 2 * DBLK; tt += 4) {
            const int qb = tt / DBLK, db = tt % DBLK;
            float *p = tile + (size_t)(32 * qb + 4 * h) * D + 32 * db + col;
#pragma unroll
            for (int r = 0; r < 16; r++) unsafeAtomicAdd(p + (8 * (r >> 2) + (r & 3)) * D, 1.0f);
        }
    }
}

hipError_t debug_atomic_tiles(float *buf, int n_slots, int tiles, int blocks, hipStream_t stream)
{
    hipLaunchKernelGGL(dbg_atomic_tiles_kernel<128>, dim3(blocks), dim3(256), 0, stream, buf,
                       n_slots, tiles);
    return hipGetLastError();
}
#endif

// Backward workspace of fa_bwd_noalloc, for callers that cannot allocate
// device memory: one copy of this array per device, held until the process
// ends.  Host code never uses its name as an address: the device address
// comes from hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void **ptr)
{
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_bwd(const BwdArgs &a)
{
    if (a.d == 128) return a.causal ? launch_bwd_t<128, true>(a) : launch_bwd_t<128, false>(a);
    return a.causal ? launch_bwd_t<64, true>(a) : launch_bwd_t<64, false>(a);
}

}  // namespace fa
