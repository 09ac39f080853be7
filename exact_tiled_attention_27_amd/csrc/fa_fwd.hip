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
// gfx950 mapping (one workgroup = 4 waves = BM = 128 query rows of one head,
// two workgroups per CU):
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
#include "fa_launch.hpp"
#include "fa_tiles.hpp"

#ifndef FA_FWD_MIN_WAVES
#define FA_FWD_MIN_WAVES 2  // waves per SIMD the register allocation must allow
#endif

namespace fa {

template <int D>
struct FwdShape {
    static constexpr int BM = 128;           // query rows per workgroup
    static constexpr int BN = 64;            // keys per tile
    static constexpr int THREADS = 256;      // 4 waves
    static constexpr int KSTEPS = D / 16;    // k-steps of S^T = K Q^T
    static constexpr int DBLK = D / 32;      // 32-row blocks of O^T
    static constexpr int NKB = BN / 32;      // 32-key blocks of S^T
    static constexpr int KVSTEPS = BN / 16;  // k-steps of O^T += V^T P^T
    using KTile = DmaTile<BN, D, THREADS>;  // row-major K tile
    using VTile = DmaTile<BN, D, THREADS>;  // row-major V tile
    static constexpr int K_BYTES = KTile::BYTES;
    static constexpr int BUF_BYTES = KTile::BYTES + VTile::BYTES;
    static constexpr int LDS_BYTES = 2 * BUF_BYTES;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, FA_FWD_MIN_WAVES) void fwd_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, float *__restrict__ o, float *__restrict__ lse, int Hq,
    int Hkv, int N, int BH, int QT, float scale_log2, float tau)
{
    using S = FwdShape<D>;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, col = lane & 31;
    const int g16 = lane >> 4;  // 16-lane group

    int bh, qt;
    xcd_tile_map(blockIdx.x, BH, QT, CAUSAL, bh, qt);
    const int b = bh / Hq, hq = bh % Hq;
    const int g = hq / (Hq / Hkv);
    const int q0 = qt * S::BM;
    const int qw0 = q0 + wave * 32;  // first query row of this wave
    const int qrow = qw0 + col;      // the query column this lane owns

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
    float l_part = 0.f;       // this lane's part of the row sum

    const int n_tiles_all = (N + S::BN - 1) / S::BN;
    const int n_tiles = CAUSAL ? min(n_tiles_all, (min(q0 + S::BM, N) + S::BN - 1) / S::BN)
                               : n_tiles_all;
    // Tiles every key of which is < N and (causal) <= q0 need no mask.
    const int n_full = CAUSAL ? min(N / S::BN, (q0 + 1) / S::BN) : N / S::BN;

    typename S::KTile kst;
    typename S::VTile vst;
    kst.init(wave, lane);
    vst.init(wave, lane);
    auto issue = [&](int tile, char *buf) {
        kst.issue(kh, tile * S::BN, N, buf, wave);
        vst.issue(vh, tile * S::BN, N, buf + S::K_BYTES, wave);
    };
    issue(0, smem);
    dma_barrier();

    auto step = [&](auto masked, int t) {
        constexpr bool MASK = decltype(masked)::value;
        const int key0 = t * S::BN;
        // The buffer for tile t + 1 was last read in step t - 1, which every
        // wave has finished (barrier at the end of that step).
        if (t + 1 < n_tiles) issue(t + 1, smem + ((t + 1) & 1) * S::BUF_BYTES);
        const char *kl = smem + (t & 1) * S::BUF_BYTES;
        const char *vl = kl + S::K_BYTES;

        // Waves whose rows all precede this tile see only masked keys: skip.
        if (!MASK || !CAUSAL || key0 <= qw0 + 31) {
            // k-step outer: each step's two K reads feed two independent chains.
            f32x16 st[S::NKB];
#pragma unroll
            for (int kb = 0; kb < S::NKB; kb++)
#pragma unroll
                for (int r = 0; r < 16; r++) st[kb][r] = 0.f;
#pragma unroll
            for (int s = 0; s < S::KSTEPS; s++)
#pragma unroll
                for (int kb = 0; kb < S::NKB; kb++)
                    st[kb] = mfma32(lds_read_bf16x8(kl, koff[s] + kb * 32 * D * 2), qf[s], st[kb]);
            if (MASK) {
#pragma unroll
                for (int kb = 0; kb < S::NKB; kb++)
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                        const bool dead = key >= N || (CAUSAL && key > qrow);
                        st[kb][r] = dead ? -INFINITY : st[kb][r];
                    }
            }
            // Tile row maximum (raw scores), in-lane then across the halves.
            float mx = st[0][0];
#pragma unroll
            for (int kb = 0; kb < S::NKB; kb++)
#pragma unroll
                for (int r = 0; r < 16; r++) mx = fmaxf(mx, st[kb][r]);
            mx = fmaxf(mx, swap_halves(mx));
            const float mt = mx * scale_log2;  // scale_log2 > 0, so max commutes

            // Conditional rescale: move the reference only when the tile max
            // exceeds it by more than tau; otherwise exponents stay <= 2^tau.
            const bool grow = mt > m_ref + tau;
            if (__any(grow)) {
                const float alpha = grow ? exp2_hw(m_ref - mt) : 1.f;
                m_ref = grow ? mt : m_ref;
                l_part *= alpha;
#pragma unroll
                for (int db = 0; db < S::DBLK; db++)
#pragma unroll
                    for (int r = 0; r < 16; r++) acc[db][r] *= alpha;
            }
            const float msub = (m_ref == -INFINITY) ? 0.f : m_ref;

            // P = exp2(s * scale * log2 e - m), row sum, bf16 B operands.
            bf16x8 pf[S::KVSTEPS];
#pragma unroll
            for (int kb = 0; kb < S::NKB; kb++) {
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const float p = exp2_hw(__builtin_fmaf(st[kb][r], scale_log2, -msub));
                    st[kb][r] = p;
                    l_part += p;
                }
                pf[2 * kb] = pack_half(st[kb], 0);
                pf[2 * kb + 1] = pack_half(st[kb], 1);
            }

            // O^T += V^T P^T.
#pragma unroll
            for (int ks = 0; ks < S::KVSTEPS; ks++)
#pragma unroll
                for (int db = 0; db < S::DBLK; db++) {
                    const i16x4 lo = lds_read_tr16(vl, voff[db][0] + 16 * ks * D * 2);
                    const i16x4 hi = lds_read_tr16(vl, voff[db][1] + 16 * ks * D * 2);
                    acc[db] = mfma32(join_bf16x8(lo, hi), pf[ks], acc[db]);
                }
        }

        dma_barrier();  // tile t + 1 has landed in LDS; tile t is no longer read
    };

    int t = 0;
    for (; t < n_full; t++) step(std::false_type{}, t);
    for (; t < n_tiles; t++) step(std::true_type{}, t);

    // Epilogue: O = O / l, LSE = (m + log2 l) * ln 2.
    const float l_tot = l_part + swap_halves(l_part);
    const float inv = 1.f / l_tot;
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

template <int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs &a)
{
    using S = FwdShape<D>;
    (void)hipGetLastError();  // clear an error left by an earlier, unrelated call
    const int QT = (a.N + S::BM - 1) / S::BM;
    const int BH = a.B * a.Hq;
    auto kern = fwd_kernel<D, CAUSAL>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(BH * QT), dim3(S::THREADS), S::LDS_BYTES, a.stream,
                       (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v, a.o,
                       a.lse, a.Hq, a.Hkv, a.N, BH, QT, a.scale * kLog2e, a.tau);
    return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs &a)
{
    if (a.d == 128) return a.causal ? launch_fwd_t<128, true>(a) : launch_fwd_t<128, false>(a);
    return a.causal ? launch_fwd_t<64, true>(a) : launch_fwd_t<64, false>(a);
}

}  // namespace fa
