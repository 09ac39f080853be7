// fa_bwd.hip -- backward exact attention for gfx950 (MI355X).
//
// Gradients of O = softmax(Q K^T * scale) V (the pages give no backward
// formulas; these are the analytic ones).  With P recomputed from the
// forward's log-sum-exp, P_ij = exp(scale * q_i . k_j - LSE_i):
//   dV_j = sum_i P_ij dO_i            dP_ij = dO_i . v_j
//   D_i  = sum_c dO_ic O_ic           dS_ij = P_ij (dP_ij - D_i)
//   dK_j = scale * sum_i dS_ij q_i    dQ_i  = scale * sum_j dS_ij k_j
// dQ is summed with fp32 global atomic adds, or in a separate pass that owns
// each dQ row (reproducible), the trade the FlashAttention-4 summary page
// describes under Limitations (deterministic backward) and Key Contributions
// item 3 (fewer dQ atomics).
//
// Kernels (all on the caller's stream, in order):
//   1. bwd_pre:   D_i, LSE_i * log2(e) per row; zero dQ in atomic mode.
//   2. bwd_dkdv:  one workgroup per (batch, kv head, 128 keys); each of the 4
//                 waves keeps 32 keys' K and V in registers and dK^T, dV^T
//                 accumulators, and walks 64-query tiles of every query head
//                 of the group.  S = Q K^T and dP = dO V^T put one key per lane
//                 (accumulator layout), so P and dS feed dV^T += dO^T P and
//                 dK^T += Q^T dS as B operands straight from registers.  In
//                 atomic mode dS goes through LDS and the workgroup adds
//                 dS K into dQ with global atomics.
//   3. bwd_dq:    (deterministic mode) one workgroup per (batch, query head,
//                 128 queries) walks the key tiles, recomputes S^T, P^T,
//                 dP^T = V dO^T, dS^T, and accumulates dQ^T += K^T dS^T in
//                 registers; one plain store per element.
#include "fa_device.hpp"
#include "fa_launch.hpp"
#include "fa_tiles.hpp"

#ifndef FA_BWD_MIN_WAVES
#define FA_BWD_MIN_WAVES 1  // waves per SIMD the dK/dV kernel's registers must allow
#endif
#ifndef FA_DQ_MIN_WAVES
#define FA_DQ_MIN_WAVES 1   // waves per SIMD the deterministic dQ kernel's registers must allow
#endif

namespace fa {

// ---------------------------------------------------------------- preprocess
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t *__restrict__ dout,
                                                      const float *__restrict__ o,
                                                      const float *__restrict__ lse,
                                                      float *__restrict__ delta,
                                                      float *__restrict__ lse2,
                                                      float *__restrict__ dq, size_t rows,
                                                      int zero_dq)
{
    constexpr int TPR = D / 8;  // threads per row, 8 elements each
    const size_t row = (size_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
    const int part = threadIdx.x % TPR;
    float acc = 0.f;
    if (row < rows) {
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
    if (row < rows && part == 0) {
        delta[row] = acc;
        lse2[row] = lse[row] * kLog2e;
    }
}

// ------------------------------------------------------------- dK/dV kernel
template <int D>
struct DkdvShape {
    static constexpr int BN = 128;   // keys per workgroup (32 per wave)
    static constexpr int BM = 64;    // queries per step
    static constexpr int THREADS = 256;
    static constexpr int KSTEPS = D / 16;
    static constexpr int DBLK = D / 32;
    using QTile = ColTile<BM, D, THREADS, true>;     // Q^T (and Q row-major from the same registers)
    using KTile = ColTile<BN, D, THREADS, false>;    // K^T, natural key order (dQ = dS K)
    static constexpr int OFF_Q = 0;                          // Q   row-major [BM][D]
    static constexpr int OFF_QT = OFF_Q + BM * D * 2;        // Q^T [D][BM]
    static constexpr int OFF_DO = OFF_QT + BM * D * 2;       // dO  row-major
    static constexpr int OFF_DOT = OFF_DO + BM * D * 2;      // dO^T
    static constexpr int OFF_DS = OFF_DOT + BM * D * 2;      // dS  row-major [BM][BN] bf16
    static constexpr int OFF_KT = OFF_DS + BM * BN * 2;      // K^T [D][BN]
    static constexpr int OFF_ROW = OFF_KT + BN * D * 2;      // lse2[BM], delta[BM]
    static constexpr int LDS_BYTES = OFF_ROW + 2 * BM * 4;
};

template <int D, bool CAUSAL, bool ATOMIC_DQ>
__global__ __launch_bounds__(256, FA_BWD_MIN_WAVES) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ dout,
    const float *__restrict__ lse2, const float *__restrict__ delta, float *__restrict__ dq,
    float *__restrict__ dk, float *__restrict__ dv, int Hq, int Hkv, int N, int BHkv, int KT,
    float scale, float scale_log2)
{
    using S = DkdvShape<D>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, col = lane & 31;

    int bg, kt;
    xcd_tile_map(blockIdx.x, BHkv, KT, false, bg, kt);
    const int b = bg / Hkv, g = bg % Hkv;
    const int grp = Hq / Hkv;
    const int kv0 = kt * S::BN;
    const int kw0 = kv0 + wave * 32;
    const int key = kw0 + col;  // the key this lane owns in S / dP / dS

    const uint16_t *kh = k + ((size_t)b * Hkv + g) * N * D;
    const uint16_t *vh = v + ((size_t)b * Hkv + g) * N * D;

    // K and V rows of this lane's key as B operands (K^T / V^T k-slices).
    bf16x8 kf[S::KSTEPS], vf[S::KSTEPS];
#pragma unroll
    for (int s = 0; s < S::KSTEPS; s++) {
        kf[s] = __builtin_bit_cast(bf16x8, gload16(kh, ((size_t)key * D + 16 * s + 8 * h) * 2, key < N));
        vf[s] = __builtin_bit_cast(bf16x8, gload16(vh, ((size_t)key * D + 16 * s + 8 * h) * 2, key < N));
    }
    if (ATOMIC_DQ) {
        typename S::KTile kt_tile;
        kt_tile.load(kh, kv0, N, tid);
        kt_tile.store(smem + S::OFF_KT, tid);
    }

    f32x16 dva[S::DBLK], dka[S::DBLK];
#pragma unroll
    for (int db = 0; db < S::DBLK; db++)
#pragma unroll
        for (int r = 0; r < 16; r++) dva[db][r] = dka[db][r] = 0.f;

    // Offsets of the A-operand reads.
    uint32_t rowoff[S::KSTEPS];  // row-major [BM][D] tile, row col (+32 qb), chunk 2s + h
#pragma unroll
    for (int s = 0; s < S::KSTEPS; s++) rowoff[s] = row_tile_off(col, 2 * s + h, D);
    uint32_t coloff[4][2];       // transposed [D][BM] tile, row 32 p + col, chunk 2 ks + h
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
#pragma unroll
        for (int p = 0; p < 2; p++) coloff[ks][p] = col_tile_off<S::BM>(32 * p + col, 2 * ks + h);

    const int first_qt = CAUSAL ? kv0 / S::BM : 0;
    const int n_qt = (N + S::BM - 1) / S::BM;
    const int steps_per_head = n_qt - first_qt;
    const int n_steps = grp * steps_per_head;  // (query head of the group, query tile) pairs
    typename S::QTile qtile, dotile;
    float *rowbuf = reinterpret_cast<float *>(smem + S::OFF_ROW);
    float row_l2 = INFINITY, row_dl = 0.f;  // this thread's lse2 / delta entry (tid < BM)

    // Global -> registers for step `st`; the loads stay in flight during the
    // previous step's compute.
    auto fetch = [&](int st) {
        const int hq = g * grp + st / steps_per_head;
        const int qs = (first_qt + st % steps_per_head) * S::BM;
        const size_t ho = ((size_t)b * Hq + hq) * N;
        qtile.load(q + ho * D, qs, N, tid);
        dotile.load(dout + ho * D, qs, N, tid);
        if (tid < S::BM) {
            const int qi = qs + tid;
            row_l2 = qi < N ? lse2[ho + qi] : INFINITY;  // P = 0 for rows >= N
            row_dl = qi < N ? delta[ho + qi] : 0.f;
        }
    };
    if (n_steps > 0) fetch(0);

    for (int st = 0; st < n_steps; st++) {
        const int hq = g * grp + st / steps_per_head;
        const int qs = (first_qt + st % steps_per_head) * S::BM;
        const size_t head_off = ((size_t)b * Hq + hq) * N;
        {
            lds_barrier();  // every wave is done with the previous step's LDS tiles
            qtile.store_rows(smem + S::OFF_Q, tid);
            qtile.store(smem + S::OFF_QT, tid);
            dotile.store_rows(smem + S::OFF_DO, tid);
            dotile.store(smem + S::OFF_DOT, tid);
            if (tid < S::BM) {
                rowbuf[tid] = row_l2;
                rowbuf[S::BM + tid] = row_dl;
            }
            lds_barrier();
            if (st + 1 < n_steps) fetch(st + 1);

            // S = Q K^T and dP = dO V^T, rows = queries, one key column per lane.
            f32x16 sc[2], dp[2];
#pragma unroll
            for (int qb = 0; qb < 2; qb++) {
#pragma unroll
                for (int r = 0; r < 16; r++) sc[qb][r] = dp[qb][r] = 0.f;
#pragma unroll
                for (int s = 0; s < S::KSTEPS; s++) {
                    const uint32_t ro = rowoff[s] + qb * 32 * D * 2;
                    sc[qb] = mfma32(lds_read_bf16x8(smem + S::OFF_Q, ro), kf[s], sc[qb]);
                    dp[qb] = mfma32(lds_read_bf16x8(smem + S::OFF_DO, ro), vf[s], dp[qb]);
                }
            }
            // P = exp2(s * scale * log2 e - LSE2), dS = P (dP - D).
            bf16x8 pf[4], dsf[4];
#pragma unroll
            for (int qb = 0; qb < 2; qb++) {
#pragma unroll
                for (int gq = 0; gq < 4; gq++) {
                    const int qr = 32 * qb + 8 * gq + 4 * h;  // rows qr .. qr+3 of the tile
                    const f32x4 l2 = lds_read_f32x4(smem + S::OFF_ROW, qr * 4);
                    const f32x4 dl = lds_read_f32x4(smem + S::OFF_ROW, (S::BM + qr) * 4);
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int r = 4 * gq + i;
                        const int qi = qs + qr + i;
                        float p = exp2_hw(__builtin_fmaf(sc[qb][r], scale_log2, -l2[i]));
                        const bool dead = key >= N || (CAUSAL && key > qi);
                        p = dead ? 0.f : p;
                        sc[qb][r] = p;
                        dp[qb][r] = p * (dp[qb][r] - dl[i]);
                    }
                }
                pf[2 * qb] = pack_half(sc[qb], 0);
                pf[2 * qb + 1] = pack_half(sc[qb], 1);
                dsf[2 * qb] = pack_half(dp[qb], 0);
                dsf[2 * qb + 1] = pack_half(dp[qb], 1);
            }
            // dV^T += dO^T P,  dK^T += Q^T dS  (contraction over the tile's queries).
#pragma unroll
            for (int db = 0; db < S::DBLK; db++)
#pragma unroll
                for (int ks = 0; ks < 4; ks++) {
                    const uint32_t co = coloff[ks][db & 1] + (db >> 1) * 64 * S::BM * 2;
                    dva[db] = mfma32(lds_read_bf16x8(smem + S::OFF_DOT, co), pf[ks], dva[db]);
                    dka[db] = mfma32(lds_read_bf16x8(smem + S::OFF_QT, co), dsf[ks], dka[db]);
                }

            if (ATOMIC_DQ) {
                // dS (bf16) -> LDS row-major [BM queries][BN keys], natural key order.
                uint16_t *dsl = reinterpret_cast<uint16_t *>(smem + S::OFF_DS);
                const int kin = wave * 32 + col;  // key index within the workgroup
#pragma unroll
                for (int qb = 0; qb < 2; qb++)
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int qr = 32 * qb + 8 * (r >> 2) + 4 * h + (r & 3);
                        const __bf16 x = (__bf16)dp[qb][r];
                        const uint32_t off = qr * (S::BN * 2) + (((kin >> 3) ^ (qr & 7)) << 4) + (kin & 7) * 2;
                        dsl[off >> 1] = __builtin_bit_cast(uint16_t, x);
                    }
                lds_barrier();
                // dQ[BM x D] += dS[BM x BN] K[BN x D]; 2*DBLK tiles of 32x32 over 4 waves.
                constexpr int TILES = 2 * S::DBLK;
#pragma unroll
                for (int tt = wave; tt < TILES; tt += 4) {
                    const int qb = tt / S::DBLK, db = tt % S::DBLK;
                    f32x16 acc;
#pragma unroll
                    for (int r = 0; r < 16; r++) acc[r] = 0.f;
#pragma unroll
                    for (int ks = 0; ks < S::BN / 16; ks++) {
                        const int qr = 32 * qb + col;
                        const uint32_t ao = qr * (S::BN * 2) + (((2 * ks + h) ^ (qr & 7)) << 4);
                        const bf16x8 a = lds_read_bf16x8(smem + S::OFF_DS, ao);
                        const bf16x8 bb = lds_read_bf16x8(smem + S::OFF_KT,
                                                          col_tile_off<S::BN>(32 * db + col, 2 * ks + h));
                        acc = mfma32(a, bb, acc);
                    }
                    float *dqh = dq + head_off * D;
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int qi = qs + 32 * qb + 8 * (r >> 2) + 4 * h + (r & 3);
                        if (qi < N) unsafeAtomicAdd(dqh + (size_t)qi * D + 32 * db + col, acc[r] * scale);
                    }
                }
            }
        }
    }

    // dV = dV^T^T, dK = scale * dK^T^T: lane holds d = 32 db + 8 gq + 4 h + i of key `key`.
    if (key < N) {
        float *dvr = dv + (((size_t)b * Hkv + g) * N + key) * D;
        float *dkr = dk + (((size_t)b * Hkv + g) * N + key) * D;
#pragma unroll
        for (int db = 0; db < S::DBLK; db++)
#pragma unroll
            for (int gq = 0; gq < 4; gq++) {
                const int dd = 32 * db + 8 * gq + 4 * h;
                f32x4 a = {dva[db][4 * gq], dva[db][4 * gq + 1], dva[db][4 * gq + 2], dva[db][4 * gq + 3]};
                f32x4 c = {dka[db][4 * gq] * scale, dka[db][4 * gq + 1] * scale,
                           dka[db][4 * gq + 2] * scale, dka[db][4 * gq + 3] * scale};
                *reinterpret_cast<f32x4 *>(dvr + dd) = a;
                *reinterpret_cast<f32x4 *>(dkr + dd) = c;
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
    using KTile = ColTile<BN, D, THREADS, true>;   // K row-major + K^T in key_pos16 order
    using VTile = RowTile<BN, D, THREADS>;         // V row-major
    static constexpr int OFF_K = 0;
    static constexpr int OFF_KT = OFF_K + BN * D * 2;
    static constexpr int OFF_V = OFF_KT + BN * D * 2;
    static constexpr int BUF_BYTES = OFF_V + BN * D * 2;
    static constexpr int LDS_BYTES = 2 * BUF_BYTES;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, FA_DQ_MIN_WAVES) void bwd_dq_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ dout,
    const float *__restrict__ lse2, const float *__restrict__ delta, float *__restrict__ dq,
    int Hq, int Hkv, int N, int BH, int QT, float scale, float scale_log2)
{
    using S = DqShape<D>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, col = lane & 31;

    int bh, qt;
    xcd_tile_map(blockIdx.x, BH, QT, CAUSAL, bh, qt);
    const int b = bh / Hq, hq = bh % Hq;
    const int g = hq / (Hq / Hkv);
    const int q0 = qt * S::BM;
    const int qw0 = q0 + wave * 32;
    const int qrow = qw0 + col;
    const size_t head_off = ((size_t)b * Hq + hq) * N;

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
    const float l2 = qrow < N ? lse2[head_off + qrow] : INFINITY;
    const float dl = qrow < N ? delta[head_off + qrow] : 0.f;

    uint32_t rowoff[S::KSTEPS];
#pragma unroll
    for (int s = 0; s < S::KSTEPS; s++) rowoff[s] = row_tile_off(col, 2 * s + h, D);
    uint32_t coloff[S::BN / 16][2];
#pragma unroll
    for (int ks = 0; ks < S::BN / 16; ks++)
#pragma unroll
        for (int p = 0; p < 2; p++) coloff[ks][p] = col_tile_off<S::BN>(32 * p + col, 2 * ks + h);

    f32x16 acc[S::DBLK];
#pragma unroll
    for (int db = 0; db < S::DBLK; db++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[db][r] = 0.f;

    const int n_tiles_all = (N + S::BN - 1) / S::BN;
    const int n_tiles = CAUSAL ? min(n_tiles_all, (min(q0 + S::BM, N) + S::BN - 1) / S::BN)
                               : n_tiles_all;
    typename S::KTile kst;
    typename S::VTile vst;
    kst.load(kh, 0, N, tid);
    vst.load(vh, 0, N, tid);
    kst.store_rows(smem + S::OFF_K, tid);
    kst.store(smem + S::OFF_KT, tid);
    vst.store(smem + S::OFF_V, tid);
    __syncthreads();

    for (int t = 0; t < n_tiles; t++) {
        const int key0 = t * S::BN;
        const bool more = t + 1 < n_tiles;
        if (more) {
            kst.load(kh, key0 + S::BN, N, tid);
            vst.load(vh, key0 + S::BN, N, tid);
        }
        const char *buf = smem + (t & 1) * S::BUF_BYTES;
        if (!CAUSAL || key0 <= qw0 + 31) {
            f32x16 st[2], dpt[2];
#pragma unroll
            for (int kb = 0; kb < 2; kb++) {
#pragma unroll
                for (int r = 0; r < 16; r++) st[kb][r] = dpt[kb][r] = 0.f;
#pragma unroll
                for (int s = 0; s < S::KSTEPS; s++) {
                    const uint32_t ro = rowoff[s] + kb * 32 * D * 2;
                    st[kb] = mfma32(lds_read_bf16x8(buf + S::OFF_K, ro), qf[s], st[kb]);
                    dpt[kb] = mfma32(lds_read_bf16x8(buf + S::OFF_V, ro), df[s], dpt[kb]);
                }
            }
            bf16x8 dsf[S::BN / 16];
#pragma unroll
            for (int kb = 0; kb < 2; kb++) {
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int kk = key0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    float p = exp2_hw(__builtin_fmaf(st[kb][r], scale_log2, -l2));
                    const bool dead = kk >= N || (CAUSAL && kk > qrow);
                    p = dead ? 0.f : p;
                    dpt[kb][r] = p * (dpt[kb][r] - dl);
                }
                dsf[2 * kb] = pack_half(dpt[kb], 0);
                dsf[2 * kb + 1] = pack_half(dpt[kb], 1);
            }
            // dQ^T += K^T dS^T (contraction over the tile's keys).
#pragma unroll
            for (int db = 0; db < S::DBLK; db++)
#pragma unroll
                for (int ks = 0; ks < S::BN / 16; ks++) {
                    const uint32_t co = coloff[ks][db & 1] + (db >> 1) * 64 * S::BN * 2;
                    acc[db] = mfma32(lds_read_bf16x8(buf + S::OFF_KT, co), dsf[ks], acc[db]);
                }
        }
        if (more) {
            char *nb = smem + ((t + 1) & 1) * S::BUF_BYTES;
            kst.store_rows(nb + S::OFF_K, tid);
            kst.store(nb + S::OFF_KT, tid);
            vst.store(nb + S::OFF_V, tid);
        }
        __syncthreads();
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
template <typename K>
static hipError_t set_lds(K kern, int bytes)
{
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs &a)
{
    (void)hipGetLastError();  // clear an error left by an earlier, unrelated call
    const size_t rows = (size_t)a.B * a.Hq * a.N;
    const float scale_log2 = a.scale * kLog2e;
    {
        constexpr int RPB = 256 / (D / 8);
        const unsigned grid = (unsigned)((rows + RPB - 1) / RPB);
        hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3(grid), dim3(256), 0, a.stream,
                           (const uint16_t *)a.dout, a.o, a.lse, a.delta, a.lse2, a.dq, rows,
                           a.deterministic ? 0 : 1);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        using S = DkdvShape<D>;
        const int KT = (a.N + S::BN - 1) / S::BN;
        const int BHkv = a.B * a.Hkv;
        hipError_t e;
        if (a.deterministic) {
            auto kern = bwd_dkdv_kernel<D, CAUSAL, false>;
            if ((e = set_lds(kern, S::LDS_BYTES)) != hipSuccess) return e;
            hipLaunchKernelGGL(kern, dim3(BHkv * KT), dim3(S::THREADS), S::LDS_BYTES, a.stream,
                               (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                               (const uint16_t *)a.dout, a.lse2, a.delta, a.dq, a.dk, a.dv, a.Hq,
                               a.Hkv, a.N, BHkv, KT, a.scale, scale_log2);
        } else {
            auto kern = bwd_dkdv_kernel<D, CAUSAL, true>;
            if ((e = set_lds(kern, S::LDS_BYTES)) != hipSuccess) return e;
            hipLaunchKernelGGL(kern, dim3(BHkv * KT), dim3(S::THREADS), S::LDS_BYTES, a.stream,
                               (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                               (const uint16_t *)a.dout, a.lse2, a.delta, a.dq, a.dk, a.dv, a.Hq,
                               a.Hkv, a.N, BHkv, KT, a.scale, scale_log2);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.deterministic) {
        using S = DqShape<D>;
        const int QT = (a.N + S::BM - 1) / S::BM;
        const int BH = a.B * a.Hq;
        auto kern = bwd_dq_kernel<D, CAUSAL>;
        hipError_t e;
        if ((e = set_lds(kern, S::LDS_BYTES)) != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(BH * QT), dim3(S::THREADS), S::LDS_BYTES, a.stream,
                           (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                           (const uint16_t *)a.dout, a.lse2, a.delta, a.dq, a.Hq, a.Hkv, a.N, BH,
                           QT, a.scale, scale_log2);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_bwd(const BwdArgs &a)
{
    if (a.d == 128) return a.causal ? launch_bwd_t<128, true>(a) : launch_bwd_t<128, false>(a);
    return a.causal ? launch_bwd_t<64, true>(a) : launch_bwd_t<64, false>(a);
}

}  // namespace fa
