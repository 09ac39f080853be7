// fa_fwd.hip -- forward exact attention for gfx950 (MI355X).
//
// The method (FlashAttention-4 pages): walk the keys tile by tile; per tile
// compute S = Q K^T * scale, update a running row maximum m and row sum l,
// accumulate O += P V with P = exp(S - m), and divide by l at the end
// (FlashAttention-4 Guide, "The Asymmetric Hardware Scaling Wall": the three
// phases per tile; its simulator walks key tiles the same way).  The
// accumulator is only renormalised when the running maximum grows by more
// than log2(256) = 8 in the base-2 exponent domain (FlashAttention-4 summary
// page, Key Contributions, item 2); P never goes through shared memory (the
// guide's "Register-Level Softmax Streaming").
//
// gfx950 mapping (one workgroup = 8 waves = BM = 256 query rows of one head,
// one workgroup per CU, two waves per SIMD):
//   * each wave owns 32 query rows; it computes S^T = K Q^T (keys x queries)
//     with v_mfma_f32_32x32x16_bf16, so every lane holds one query column:
//     row max and row sum are in-lane, plus one swap between the wave halves;
//   * the bf16 P^T tile, still in the accumulator layout, is the B operand of
//     O^T += V^T P^T (contraction over keys), so P stays in registers;
//   * K and V tiles are staged to LDS row-major, double-buffered and
//     XOR-swizzled; the V^T operand is read with transposing LDS loads
//     (ds_read_b64_tr_b16) in exactly the key order the P^T registers present;
//   * tiles that need no mask (all keys < N and, when causal, all keys <= the
//     workgroup's first query) run a loop body compiled without mask code;
//   * scores use the base-2 domain: x = s * (scale * log2 e) - m.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_exp2_poly.hpp"
#include "fa_launch.hpp"
#include "fa_tiles.hpp"

#ifndef FA_FWD_MIN_WAVES
#define FA_FWD_MIN_WAVES 2  // waves per SIMD the register allocation must allow
#endif

namespace fa {

#if FA_DEBUG_COUNTERS
// Debug build only: event counters of the forward kernels (indices in
// fa_launch.hpp, kDbg*), read and cleared by debug_counters().
__device__ unsigned long long dbg_counters[kDbgCount];

// Adds popcount(pred over the wave's lanes) to counter c (one atomic per wave).
__device__ __forceinline__ void dbg_count(int c, bool pred, int lane)
{
    const unsigned long long n = __popcll(__ballot(pred));
    if (lane == 0 && n) atomicAdd(&dbg_counters[c], n);
}
#endif

template <int D>
struct FwdShape {
    static constexpr int BM = 256;           // query rows per workgroup (32 per wave)
    static constexpr int BN = 64;            // keys per tile
    static constexpr int THREADS = 512;      // 8 waves: each K / V tile copied once per 256 rows
    static constexpr int KSTEPS = D / 16;    // k-steps of S^T = K Q^T
    static constexpr int DBLK = D / 32;      // 32-row blocks of O^T
    static constexpr int NKB = BN / 32;      // 32-key blocks of S^T
    static constexpr int KVSTEPS = BN / 16;  // k-steps of O^T += V^T P^T
    using KTile = DmaTile<BN, D, THREADS>;  // row-major K (and V) tile
    // LDS: two K slots and two V slots (tile t uses slot t % 2 of each), four
    // separate arrays addressed with compile-time slot numbers.  The tile
    // copies are inline-asm buffer loads the compiler does not track; the
    // step barrier waits for them.
    static constexpr int TILE_BYTES = KTile::BYTES;
};

// Software pipeline of one wave (tile t, with S_t already computed, masked,
// and its row maximum folded into the reference m):
//   1. barrier: V_t and K_{t+1} are in LDS, every wave is done with K_t and
//      V_{t-1}; start the copies of V_{t+1} and K_{t+2} into the freed slots
//      (in mask-free steps, one copy per k-step between the score products);
//   2. one straight-line block: S_{t+1} = K_{t+1} Q^T on the matrix cores,
//      P_t = exp2(S_t * c - m) with its row sum and bf16 packing on the vector
//      ALUs, then O^T += V_t^T P_t^T;
//   3. mask S_{t+1} (diagonal, tail and sliding-window edge tiles only), take
//      its row maximum and, rarely, rescale O and l.
// The exponentials of one tile thus overlap the score products of the next
// (the overlap the FlashAttention-4 guide obtains with separate softmax and
// MMA warps), inside each wave and without extra barriers.
// POLY: share of the exponentials computed by the cubic polynomial on the FMA
// units (FlashAttention-4 summary page, Key Contributions, item 2): 0 none,
// 4 one in four (score rows r % 4 == 3), 1 all.  v_exp_f32 issues at half the
// VALU rate on gfx950 and the polynomial costs about seven full-rate
// operations, so the default is none.
// SPLIT: the keys of each query tile are cut into n_splits chunks of whole
// tiles, one workgroup per (query tile, chunk); a workgroup writes its
// chunk's normalised partial O and partial LSE to opart / lpart
// ([n_splits][B * Hq][N] rows) for fwd_merge_kernel.  A row with no valid key
// in its chunk (causal) gets O = 0 and LSE = -inf there.
// window (causal only): query i sees keys i - window + 1 .. i; tiles before
// the workgroup's first such key are skipped (kNoWindow when there is none).
// BIAS: the linear position bias, slopes[hq] * (key - query) added to every
// scaled score (added here to the raw score as slope / scale * (key - query),
// before the mask and the row maximum, so everything after is unchanged).
template <int D, bool CAUSAL, int POLY, bool SPLIT, bool BIAS = false>
__global__ __launch_bounds__(512, FA_FWD_MIN_WAVES) void fwd_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, float *__restrict__ o, float *__restrict__ lse, int Hq,
    int Hkv, int N, int BH, int QT, float scale_log2, float tau, int window, int n_splits,
    float *__restrict__ opart, float *__restrict__ lpart, const float *__restrict__ slopes,
    int linear_map)
{
    using S = FwdShape<D>;
    __shared__ __attribute__((aligned(16))) char k_lds0[S::TILE_BYTES];
    __shared__ __attribute__((aligned(16))) char k_lds1[S::TILE_BYTES];
    __shared__ __attribute__((aligned(16))) char v_lds0[S::TILE_BYTES];
    __shared__ __attribute__((aligned(16))) char v_lds1[S::TILE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar LDS bases
    const int h = lane >> 5, col = lane & 31;
    const int g16 = lane >> 4;  // 16-lane group

    int bh, qt, split = 0;
    if (SPLIT) {
        int vt;  // (query tile, chunk) pairs, longest first when causal
        xcd_tile_map(blockIdx.x, BH, QT * n_splits, CAUSAL, linear_map, bh, vt);
        qt = vt / n_splits;
        split = vt % n_splits;
    } else {
        xcd_tile_map(blockIdx.x, BH, QT, CAUSAL, linear_map, bh, qt);
    }
    const int b = bh / Hq, hq = bh % Hq;
    const int g = hq / (Hq / Hkv);
    const int q0 = qt * S::BM;
    const int qrow = q0 + wave * 32 + col;  // the query column this lane owns
    const float bias_a = BIAS ? slopes[hq] * (kLog2e / scale_log2) : 0.f;  // slope / scale

    const int n_tiles_all = (N + S::BN - 1) / S::BN;
    const int n_tiles_q = CAUSAL ? min(n_tiles_all, (min(q0 + S::BM, N) + S::BN - 1) / S::BN)
                                 : n_tiles_all;
    // Causal sliding window (window >= 1; at least N means none): query i
    // sees keys i - window + 1 .. i.  t_lo: the first tile any row of the
    // workgroup sees; w_full: the first tile every row sees whole.
    const int t_lo = CAUSAL ? max(0, q0 - window + 1) / S::BN : 0;
    const int w_full = CAUSAL ? (max(0, q0 + S::BM - window) + S::BN - 1) / S::BN : 0;
    // This workgroup's key tiles [t_begin, n_tiles): all of them, or its chunk.
    int t_begin = t_lo, n_tiles = n_tiles_q;
    if (SPLIT) {
        const int per = (n_tiles_q - t_lo + n_splits - 1) / n_splits;
        t_begin = min(t_lo + split * per, n_tiles_q);
        n_tiles = min(t_begin + per, n_tiles_q);
        if (t_begin >= n_tiles) {
            // Empty chunk (more chunks than tiles): O = 0, LSE = -inf.
            if (qrow < N) {
                const size_t prow = ((size_t)split * BH + bh) * N + qrow;
                float *orow = opart + prow * D;
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int db = 0; db < S::DBLK; db++)
#pragma unroll
                    for (int gq = 0; gq < 4; gq++)
                        *reinterpret_cast<f32x4 *>(orow + db * 32 + 8 * gq + 4 * h) = z;
                if (h == 0) lpart[prow] = -INFINITY;
            }
            return;
        }
    }
    // Tiles every key of which is < N and (causal) <= q0 need no mask (and,
    // split, lie in the chunk).
    const int n_full = min(n_tiles, CAUSAL ? min(N / S::BN, (q0 + 1) / S::BN) : N / S::BN);

    const uint16_t *qh = q + ((size_t)b * Hq + hq) * N * D;
    const uint16_t *kh = k + ((size_t)b * Hkv + g) * N * D;
    const uint16_t *vh = v + ((size_t)b * Hkv + g) * N * D;

    // Q^T as B operand: lane holds Q[qrow][16 s + 8 h .. +7].
    bf16x8 qf[S::KSTEPS];
#pragma unroll
    for (int s = 0; s < S::KSTEPS; s++)
        qf[s] = __builtin_bit_cast(bf16x8, gload16(qh, ((size_t)qrow * D + 16 * s + 8 * h) * 2, qrow < N));

    // LDS byte offsets.  K (A operand of S^T): row kb*32 + col, chunk 2s + h;
    // the swizzle only sees row & 15, so kb*32 rows are an immediate offset.
    uint32_t koff[S::KSTEPS];
#pragma unroll
    for (int s = 0; s < S::KSTEPS; s++) koff[s] = tile_off(col, 2 * s + h, D);
    // V^T (A operand of O^T) by transposing reads: read rho of k-step ks covers
    // keys 16 ks + 8 rho + 4 h .. +3 (the key order of the P^T registers) and
    // head-dimension columns 32 db + (lane % 32); 16 ks rows are an immediate.
    uint32_t voff[S::DBLK][2];
#pragma unroll
    for (int db = 0; db < S::DBLK; db++)
#pragma unroll
        for (int rho = 0; rho < 2; rho++)
            voff[db][rho] = tr_off(8 * rho + 4 * h, 32 * db + 16 * (g16 & 1), lane, D);

    f32x16 acc[S::DBLK];
#pragma unroll
    for (int db = 0; db < S::DBLK; db++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[db][r] = 0.f;
    float m_ref = -INFINITY;  // reference maximum (base-2 domain) the exponent subtracts
    float l_part = 0.f;       // this lane's part of the row sum (fp32 p: the LSE)
    float w_part = 0.f;       // ... of the bf16 weights P V applies (O's divisor)


    // K and V tiles have one shape, so one set of per-lane copy offsets.
    typename S::KTile kv_dma;
    kv_dma.init(wave, lane);
    // Tile t lives in slot t % 2 of the K and of the V region.  Callers pass
    // the slot as a compile-time constant, so every LDS address is a per-lane
    // register plus an immediate.
    using Slot0 = std::integral_constant<int, 0>;
    using Slot1 = std::integral_constant<int, 1>;
    const BufRsrc krs = make_rsrc(kh, (uint32_t)N * D * 2);
    const BufRsrc vrs = make_rsrc(vh, (uint32_t)N * D * 2);
    auto issue_k = [&](int t, auto slot) {
        kv_dma.issue(krs, t * S::BN, N, decltype(slot)::value ? k_lds1 : k_lds0, wave);
    };
    auto issue_v = [&](int t, auto slot) {
        kv_dma.issue(vrs, t * S::BN, N, decltype(slot)::value ? v_lds1 : v_lds0, wave);
    };

    // S^T_t = K_t Q^T (raw scores).  k-step outer: two independent chains.
    // piece(s) runs after k-step s's products (tile copies placed in their
    // shadow).
    auto scores_with = [&](f32x16(&st)[S::NKB], auto slot, auto piece) {
        const char *kl = decltype(slot)::value ? k_lds1 : k_lds0;
#pragma unroll
        for (int s = 0; s < S::KSTEPS; s++) {
#pragma unroll
            for (int kb = 0; kb < S::NKB; kb++)
                st[kb] = mfma32(lds_read_bf16x8(kl, koff[s] + kb * 32 * D * 2), qf[s],
                                s == 0 ? f32x16{} : st[kb]);
            piece(s);
        }
    };
    auto scores = [&](f32x16(&st)[S::NKB], auto slot) { scores_with(st, slot, [](int) {}); };
    // Raw scores of tile t += slope / scale * (key - query): per lane one
    // base for the tile, per register a fixed key offset.
    auto add_bias = [&](f32x16(&st)[S::NKB], int t) {
        const float base = bias_a * (float)(t * S::BN + 4 * h - qrow);
#pragma unroll
        for (int kb = 0; kb < S::NKB; kb++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                st[kb][r] += __builtin_fmaf(bias_a, (float)(kb * 32 + 8 * (r >> 2) + (r & 3)), base);
    };
    auto apply_mask = [&](f32x16(&st)[S::NKB], int t) {
#pragma unroll
        for (int kb = 0; kb < S::NKB; kb++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int key = t * S::BN + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                const bool dead = key >= N || (CAUSAL && (key > qrow || qrow - key >= window));
                st[kb][r] = dead ? -INFINITY : st[kb][r];
            }
    };
    // Tile row maximum, then the conditional rescale: the reference moves
    // only when the tile maximum exceeds it by more than tau, otherwise the
    // exponents stay <= 2^tau.
    auto row_max_rescale = [&](f32x16(&st)[S::NKB]) {
        float mx = st[0][0];
#pragma unroll
        for (int kb = 0; kb < S::NKB; kb++)
#pragma unroll
            for (int r = 0; r < 16; r++) mx = fmaxf(mx, st[kb][r]);
        const float mt = halves_max(mx) * scale_log2;  // scale_log2 > 0: max commutes
        const bool grow = mt > m_ref + tau;
#if FA_DEBUG_COUNTERS
        {
            // One decision per live query row (lanes of the first half) and
            // tile, once the row has a reference; rows that move it; waves
            // that take the rescale branch for such a row.
            const bool decided = h == 0 && qrow < N && m_ref != -INFINITY;
            dbg_count(kDbgRowDecisions, decided, lane);
            dbg_count(kDbgRowRescales, decided && grow, lane);
            dbg_count(kDbgWaveRescales, lane == 0 && __any(decided && grow), lane);
        }
#endif
        if (__any(grow)) {
            const float alpha = grow ? exp2_hw(m_ref - mt) : 1.f;
            m_ref = grow ? mt : m_ref;
            l_part *= alpha;
            w_part *= alpha;
#pragma unroll
            for (int db = 0; db < S::DBLK; db++)
#pragma unroll
                for (int r = 0; r < 16; r++) acc[db][r] *= alpha;
        }
    };
    // P = exp2(s * scale * log2 e - m), its fp32 row sum (four short add
    // chains), the bf16 B operands, and the row sum of those bf16 values
    // (one dot product with (1, 1) per pair).  The fp32 sum gives the
    // log-sum-exp, which must not inherit bf16 rounding on short rows; the
    // bf16 sum divides O, so that O is an exact weighted mean of V rows with
    // the weights P V applied: a dominant key's rounding (up to 2^-9 of its
    // weight, whose exponent may reach tau above the reference) cancels
    // instead of scaling O.
    auto exp_pack = [&](f32x16(&st)[S::NKB], bf16x8(&pf)[S::KVSTEPS]) {
        const float msub = (m_ref == -INFINITY) ? 0.f : m_ref;
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
        float ws[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < S::NKB; kb++) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const float x = __builtin_fmaf(st[kb][r], scale_log2, -msub);
                const bool on_fma = POLY == 1 || (POLY == 4 && (r & 3) == 3);
                const float p = on_fma ? exp2_poly(x) : exp2_hw(x);
                st[kb][r] = p;
                ls[r & 3] += p;
            }
            pf[2 * kb] = pack_half(st[kb], 0);
            pf[2 * kb + 1] = pack_half(st[kb], 1);
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const u32x4 pairs = __builtin_bit_cast(u32x4, pf[2 * kb + j]);
#pragma unroll
                for (int e = 0; e < 4; e++) ws[e] = sum_bf16_pair(pairs[e], ws[e]);
            }
        }
        l_part += (ls[0] + ls[1]) + (ls[2] + ls[3]);
        w_part += (ws[0] + ws[1]) + (ws[2] + ws[3]);
    };
    // O^T += V_t^T P_t^T.
    auto pv = [&](const bf16x8(&pf)[S::KVSTEPS], auto slot) {
        const char *vl = decltype(slot)::value ? v_lds1 : v_lds0;
#pragma unroll
        for (int ks = 0; ks < S::KVSTEPS; ks++)
#pragma unroll
            for (int db = 0; db < S::DBLK; db++) {
                const i16x4 lo = lds_read_tr16(vl, voff[db][0] + 16 * ks * D * 2);
                const i16x4 hi = lds_read_tr16(vl, voff[db][1] + 16 * ks * D * 2);
                acc[db] = mfma32(join_bf16x8(lo, hi), pf[ks], acc[db]);
            }
    };
    // One pipeline step for tile t (slot P = t % 2).  NEXT: 0 = tile t + 1
    // does not exist, 1 = it needs no mask (the common case: one basic block
    // from the copies to the next row maximum), 2 = it may need a mask.
    auto step = [&](auto next_kind, auto parity, f32x16(&cur)[S::NKB], f32x16(&nxt)[S::NKB],
                    int t) {
        constexpr int NEXT = decltype(next_kind)::value;
        constexpr int P = decltype(parity)::value;
        using Here = std::integral_constant<int, P>;
        using There = std::integral_constant<int, 1 - P>;
        dma_barrier();
        bf16x8 pf[S::KVSTEPS];
        if constexpr (NEXT == 1) {
            // Full steps: tiles t + 1 (V) and t + 2 (K) are whole; their
            // copies go one per k-step between the score products.
            constexpr int PW = S::KTile::PER_WAVE;
            char *vdst = P ? v_lds0 : v_lds1;
            char *kdst = P ? k_lds1 : k_lds0;
            const bool knext = (t + 3) * S::BN <= N && t + 2 < n_tiles;  // whole tile
            if (!knext && t + 2 < n_tiles) issue_k(t + 2, Here{});
            scores_with(nxt, There{}, [&](int s) {
                if (s < PW)
                    kv_dma.issue_block(vrs, (t + 1) * S::BN, vdst, wave, s);
                else if (s < 2 * PW && knext)
                    kv_dma.issue_block(krs, (t + 2) * S::BN, kdst, wave, s - PW);
            });
        } else {
            if (NEXT) issue_v(t + 1, There{});
            if (t + 2 < n_tiles) issue_k(t + 2, Here{});
            if (NEXT) scores(nxt, There{});
        }
        exp_pack(cur, pf);
        pv(pf, Here{});
        if (BIAS && NEXT) add_bias(nxt, t + 1);
        if (NEXT == 2 && (t + 1 >= n_full || t + 1 < w_full)) apply_mask(nxt, t + 1);
        if (NEXT) row_max_rescale(nxt);
    };
    using Last = std::integral_constant<int, 0>;
    using Full = std::integral_constant<int, 1>;
    using Any = std::integral_constant<int, 2>;

#if FA_DEBUG_COUNTERS
    // Key tiles this workgroup walks, and how many of them take the masked
    // path (diagonal, tail and window-edge tiles).
    if (tid == 0) {
        atomicAdd(&dbg_counters[kDbgTiles], (unsigned long long)(n_tiles - t_begin));
        int masked = 0;
        for (int t = t_begin; t < n_tiles; t++) masked += (t >= n_full || t < w_full);
        atomicAdd(&dbg_counters[kDbgMaskedTiles], (unsigned long long)masked);
        atomicAdd(&dbg_counters[kDbgWorkgroups], 1ull);
    }
#endif
    // Prologue: K_0, V_0, K_1 copied while the Q loads are in flight (the
    // barrier drains both; the loads are settled right after it, so none is
    // still counted when the loop's copies start); S_0.
    f32x16 sa[S::NKB], sb[S::NKB];
    issue_k(t_begin, Slot0{});
    issue_v(t_begin, Slot0{});
    if (t_begin + 1 < n_tiles) issue_k(t_begin + 1, Slot1{});
    dma_barrier();
#pragma unroll
    for (int s = 0; s < S::KSTEPS; s++) settle(qf[s]);
    scores(sa, Slot0{});
    if (BIAS) add_bias(sa, t_begin);
    if (n_full <= t_begin || t_begin < w_full) apply_mask(sa, t_begin);
    row_max_rescale(sa);

    // Unrolled by two: the score registers and LDS slots alternate statically.
    // Steps whose next tile is unmasked first, then the (at most a few)
    // diagonal and tail tiles.
    int t = t_begin;
    // Sliding window: leading tiles the window cuts for some rows.
    for (; t + 2 < n_tiles && t + 1 < w_full; t += 2) {
        step(Any{}, Slot0{}, sa, sb, t);
        step(Any{}, Slot1{}, sb, sa, t + 1);
    }
    for (; t + 2 < n_full; t += 2) {
        step(Full{}, Slot0{}, sa, sb, t);
        step(Full{}, Slot1{}, sb, sa, t + 1);
    }
    for (; t + 2 < n_tiles; t += 2) {
        step(Any{}, Slot0{}, sa, sb, t);
        step(Any{}, Slot1{}, sb, sa, t + 1);
    }
    if (t + 1 < n_tiles) {
        step(Any{}, Slot0{}, sa, sb, t);
        step(Last{}, Slot1{}, sb, sb, t + 1);
    } else {
        step(Last{}, Slot0{}, sa, sa, t);
    }

    // Epilogue: O = O / w (the bf16 weights' sum), LSE = (m + log2 l) * ln 2.
    const float l_tot = halves_sum(l_part);
    const float w_tot = halves_sum(w_part);
    if (SPLIT) {
        if (qrow < N) {
            const size_t prow = ((size_t)split * BH + bh) * N + qrow;
            float *orow = opart + prow * D;
            const float inv = w_tot > 0.f ? 1.f / w_tot : 0.f;  // no valid key: O = 0
#pragma unroll
            for (int db = 0; db < S::DBLK; db++)
#pragma unroll
                for (int gq = 0; gq < 4; gq++) {
                    f32x4 val = {acc[db][4 * gq] * inv, acc[db][4 * gq + 1] * inv,
                                 acc[db][4 * gq + 2] * inv, acc[db][4 * gq + 3] * inv};
                    *reinterpret_cast<f32x4 *>(orow + db * 32 + 8 * gq + 4 * h) = val;
                }
            if (h == 0) lpart[prow] = l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
        }
        return;
    }
    const float inv = 1.f / w_tot;
    if (qrow < N) {
        float *orow = o + (((size_t)b * Hq + hq) * N + qrow) * D;
#pragma unroll
        for (int db = 0; db < S::DBLK; db++)
#pragma unroll
            for (int gq = 0; gq < 4; gq++) {
                f32x4 val = {acc[db][4 * gq] * inv, acc[db][4 * gq + 1] * inv,
                             acc[db][4 * gq + 2] * inv, acc[db][4 * gq + 3] * inv};
                *reinterpret_cast<f32x4 *>(orow + db * 32 + 8 * gq + 4 * h) = val;
            }
        if (lse && h == 0) lse[((size_t)b * Hq + hq) * N + qrow] = (m_ref + log2f(l_tot)) * kLn2;
    }
}

// Merge of the split-KV partial results, one row per D / 4 threads: with
// M = max_s LSE_s and w_s = exp(LSE_s - M), O = sum_s w_s O_s / sum_s w_s and
// LSE = M + ln sum_s w_s, the log-sum-exp over the union of the chunks' keys
// (each O_s is normalised by its own chunk's sum).  Chunk 0 holds key 0,
// valid for every row, so M is finite and sum_s w_s >= 1.
template <int D>
__global__ __launch_bounds__(256) void fwd_merge_kernel(const float *__restrict__ opart,
                                                        const float *__restrict__ lpart,
                                                        float *__restrict__ o,
                                                        float *__restrict__ lse, size_t rows,
                                                        int n_splits)
{
    constexpr int TPR = D / 4;  // threads per row, 4 values each
    const size_t row = (size_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
    const int part = threadIdx.x % TPR;
    if (row >= rows) return;
    float m = -INFINITY;
    for (int s = 0; s < n_splits; s++) m = fmaxf(m, lpart[(size_t)s * rows + row]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    for (int s = 0; s < n_splits; s++) {
        const float w = exp2_hw((lpart[(size_t)s * rows + row] - m) * kLog2e);  // -inf -> 0
        const f32x4 x = *reinterpret_cast<const f32x4 *>(opart + ((size_t)s * rows + row) * D + 4 * part);
        acc += w * x;
        wsum += w;
    }
    *reinterpret_cast<f32x4 *>(o + row * D + 4 * part) = acc * (1.f / wsum);
    if (lse && part == 0) lse[row] = m + logf(wsum);
}

template <int D, bool CAUSAL, bool SPLIT>
static hipError_t launch_fwd_split(const FwdArgs &a)
{
    using S = FwdShape<D>;
    const int QT = (a.N + S::BM - 1) / S::BM;
    const int BH = a.B * a.Hq;
    auto kern = a.poly == 1 ? fwd_kernel<D, CAUSAL, 1, SPLIT>
              : a.poly == 4 ? fwd_kernel<D, CAUSAL, 4, SPLIT>
                            : fwd_kernel<D, CAUSAL, 0, SPLIT>;
    // The bias has one instance: exponentials on v_exp_f32, one pass.
    if (!SPLIT && a.slopes) kern = fwd_kernel<D, CAUSAL, 0, SPLIT, !SPLIT>;
    const int splits = SPLIT ? a.splits : 1;
    hipLaunchKernelGGL(kern, dim3(BH * QT * splits), dim3(S::THREADS), 0, a.stream,
                       (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v, a.o,
                       a.lse, a.Hq, a.Hkv, a.N, BH, QT, a.scale * kLog2e, a.tau,
                       a.window > 0 ? a.window : kNoWindow, splits, a.opart, a.lpart, a.slopes,
                       a.linear_map);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !SPLIT) return e;
    const size_t rows = (size_t)BH * a.N;
    constexpr int RPB = 256 / (D / 4);  // rows per merge block
    hipLaunchKernelGGL(fwd_merge_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                       a.stream, a.opart, a.lpart, a.o, a.lse, rows, splits);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs &a)
{
    (void)hipGetLastError();  // clear an error left by an earlier, unrelated call
    return a.splits > 1 ? launch_fwd_split<D, CAUSAL, true>(a) : launch_fwd_split<D, CAUSAL, false>(a);
}

#if FA_DEBUG_COUNTERS
hipError_t debug_counters(unsigned long long *host, int n)
{
    unsigned long long zero[kDbgCount] = {};
    hipError_t e = hipMemcpyFromSymbol(host, HIP_SYMBOL(dbg_counters),
                                       sizeof(unsigned long long) * (n < kDbgCount ? n : kDbgCount));
    if (e != hipSuccess) return e;
    return hipMemcpyToSymbol(HIP_SYMBOL(dbg_counters), zero, sizeof zero);
}
#endif

hipError_t launch_fwd(const FwdArgs &a)
{
    if (a.d == 128) return a.causal ? launch_fwd_t<128, true>(a) : launch_fwd_t<128, false>(a);
    return a.causal ? launch_fwd_t<64, true>(a) : launch_fwd_t<64, false>(a);
}

}  // namespace fa
