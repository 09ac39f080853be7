/*
 * fa.h -- C ABI of the MI355X (gfx950) exact tiled attention library libfa.so.
 *
 * What the calls compute:
 *   Forward: per tile of keys, S = Q K^T * scale, a running row max / row sum
 *   softmax P = exp(S - m) / l, and O = P V (page "FlashAttention-4 Guide:
 *   Kernel Pipelining on Blackwell", section "The Asymmetric Hardware Scaling
 *   Wall": three phases per tile; its simulator in "End-to-End
 *   Implementation" walks key tiles with a running max and sum).  The result
 *   is exact attention softmax(Q K^T * scale) V up to rounding.  The
 *   normalisation is skipped unless the running maximum grows by more than
 *   log2(256) = 8 in the base-2 exponent domain (page "FlashAttention-4",
 *   section "Key Contributions", item 2).
 *   Backward: dQ, dK, dV of the same function, with P recomputed from the
 *   saved log-sum-exp; dQ is summed with global atomic adds, by a separate
 *   deterministic pass, or with the atomic adds put in a fixed order (page
 *   "FlashAttention-4", "Key Contributions" item 3 and "Limitations": the
 *   deterministic mode trades speed for reproducibility).
 *
 * Conventions shared by every call:
 *   - Tensors are device pointers to dense row-major arrays laid out
 *     [B, H, N, d] (sequence-major within a head, as in the simulator's
 *     [Batch, Heads, Len, HeadDim]).  Q, dO, O, dQ use H = Hq; K, V, dK, dV use
 *     H = Hkv.  LSE is [B, Hq, N].
 *   - bf16 tensors hold IEEE bfloat16 bit patterns (uint16).  O, LSE, dQ, dK,
 *     dV are float32.
 *   - Grouped-query attention: query head h reads key/value head
 *     h / (Hq / Hkv).
 *   - causal != 0 keeps key j for query i iff j <= i.
 *   - LSE is the natural-log log-sum-exp of the scaled scores of each row:
 *     LSE_i = ln sum_j exp(scale * q_i . k_j).
 *   - The caller owns every buffer; the library allocates no device memory,
 *     keeps no state between calls and may be called concurrently on
 *     different streams with disjoint outputs.  The one exception is
 *     fa_bwd_noalloc, whose workspace is a static device array of the
 *     library shared by all its calls on a device (see there).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     without any host synchronisation.  Argument errors return before any
 *     work is enqueued.  A launch failure returns FA_ERR_HIP; faults during
 *     execution surface at the caller's next synchronisation.
 *   - The environment variable FA_EXP2_POLY, read on every forward call
 *     (fa_fwd, fa_fwd_window, fa_fwd_splitkv, fa_fwd_alibi),
 *     moves forward exponentials from the transcendental unit to a cubic
 *     polynomial on the FMA units (page "FlashAttention-4", Key Contributions
 *     item 2): "1" all of them, "4" one in four; unset or any other value,
 *     none (the default, and the faster choice on this chip).  The
 *     polynomial's relative error is at most 7.5e-5 (a minimax fit below
 *     bf16's half ulp), and it clamps its argument at -127: masked scores
 *     (-inf) and scores more than 127 below the row's reference contribute
 *     2^-127 each instead of 0, which is below fp32 rounding of a row sum
 *     that is at least 1.
 *   - The environment variable FA_RESCALE_TAU, read on every forward call,
 *     replaces the rescale threshold 8 by another finite value >= 0 (0:
 *     rescale whenever the running maximum grows); the result is the same
 *     up to rounding.
 *   - The environment variable FA_WORKGROUP_ORDER, read on every call, set
 *     to "linear" launches workgroups in plain head-major order instead of
 *     grouping each head's workgroups on one XCD (and, with the causal mask,
 *     issuing the longest query tiles first), for measuring what the
 *     default order gains.  Every workgroup computes the same values either
 *     way, so the outputs are the same bits (apart from dQ in FA_BWD_ATOMIC
 *     mode, whose order of additions is unspecified in any case).
 *   - The environment variable FA_PAIR_PATH, read on every backward call,
 *     set to "memory" makes FA_BWD_ATOMIC_PAIRED hand its partial dQ tiles
 *     over through memory (device-scope stores and loads) for every pair,
 *     not only for pairs whose workgroups run on different XCDs: the same
 *     sums, for testing that path and measuring what the L2 path gains.
 *   - The environment variable FA_WAIT_TICKS, read on every backward call,
 *     replaces the longest wait of FA_BWD_ORDERED and FA_BWD_ATOMIC_PAIRED
 *     for another workgroup (2 s) by that many ticks of the 100 MHz wall
 *     clock (an integer >= 0; 0: a wait whose condition is not met at once
 *     gives up): for testing the timeout path described at
 *     fa_bwd_workspace_bytes.
 *   - Supported: d in {64, 128}; B, Hq, Hkv, N >= 1; Hq % Hkv == 0;
 *     scale > 0 and finite; every pointer 16-byte aligned; N need not be a
 *     multiple of any tile size; one head's bf16 rows, N * d * 2 bytes, must
 *     stay below 2 GiB (N < 8388608 at d = 128).  Element offsets are 64-bit.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,        /* a required pointer is NULL                       */
    FA_ERR_SHAPE = 2,       /* B/Hq/Hkv/N < 1, Hq % Hkv != 0, N too large,
                               scale invalid, or window, split count or dQ
                               mode out of range                               */
    FA_ERR_UNSUPPORTED = 3, /* head dimension d not in {64, 128}                */
    FA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                 */
    FA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required       */
    FA_ERR_HIP = 6          /* the HIP runtime reported an error on launch      */
} fa_status;

/*
 * Forward attention.
 *   q   bf16 [B, Hq,  N, d]   (read)
 *   k   bf16 [B, Hkv, N, d]   (read)
 *   v   bf16 [B, Hkv, N, d]   (read)
 *   o   fp32 [B, Hq,  N, d]   (written: softmax(q k^T * scale) v)
 *   lse fp32 [B, Hq,  N]      (written; may be NULL when not needed)
 * Returns an fa_status.
 */
int fa_fwd(const void *q, const void *k, const void *v, float *o, float *lse,
           int B, int Hq, int Hkv, int N, int d, float scale, int causal, void *stream);

/*
 * Causal sliding-window forward: query i attends to keys
 * max(0, i - window + 1) .. i only, the banded mask of local attention (the
 * page "FlashAttention-4 Guide: Kernel Pipelining on Blackwell", section
 * "Production Deployment Guide", points to custom masks of this kind; the
 * pages give no formula, so the band is the reading stated here).  Key tiles
 * wholly outside the band are skipped.  window >= 1 (window >= N is plain
 * causal attention); otherwise FA_ERR_SHAPE.  Other arguments and outputs as
 * in fa_fwd; the LSE runs over the row's band.
 * Returns an fa_status.
 */
int fa_fwd_window(const void *q, const void *k, const void *v, float *o, float *lse,
                  int B, int Hq, int Hkv, int N, int d, float scale, int window, void *stream);

/*
 * Split-KV forward: the same result as fa_fwd (up to rounding), computed with
 * the keys of every query tile cut into num_splits chunks that separate
 * workgroups process, each writing a partial O normalised by its own row
 * sums and a partial LSE; a merge pass then combines them per row as
 * O = sum_s w_s O_s / sum_s w_s, LSE = M + ln sum_s w_s with
 * w_s = exp(LSE_s - M), M = max_s LSE_s.  The combination is the identity of
 * the online softmax (the running max and sum of the page "FlashAttention-4
 * Guide: Kernel Pipelining on Blackwell", "The Asymmetric Hardware Scaling
 * Wall") applied to whole chunks instead of single tiles.  It pays when
 * B * Hq * ceil(N / 256) workgroups leave the chip's compute units idle
 * (few heads, long sequences).
 *   num_splits: 1 .. FA_MAX_SPLITS; 1 is fa_fwd itself (no workspace needed).
 *   workspace / workspace_bytes: device scratch of at least
 *     fa_fwd_splitkv_workspace_bytes(...) bytes, 16-byte aligned, owned by
 *     the caller, contents ignored on entry: the partial O
 *     ([num_splits][B * Hq][N][d] fp32) and partial LSE
 *     ([num_splits][B * Hq][N] fp32), each rounded up to 256 bytes.
 *   Other arguments and outputs as in fa_fwd; num_splits outside the range
 *   returns FA_ERR_SHAPE.
 * Returns an fa_status.
 */
#define FA_MAX_SPLITS 64
int fa_fwd_splitkv(const void *q, const void *k, const void *v, float *o, float *lse,
                   int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                   int num_splits, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of workspace fa_fwd_splitkv needs; 0 when num_splits == 1 or for an
 * invalid shape or split count.
 */
size_t fa_fwd_splitkv_workspace_bytes(int B, int Hq, int Hkv, int N, int d, int num_splits);

/*
 * dQ modes of fa_bwd (its `deterministic` argument).
 *   FA_BWD_ATOMIC:   the dK/dV kernel adds each key block's dS K into dq
 *                    with fp32 atomic adds in whatever order they land
 *                    (bits may differ from run to run).
 *   FA_BWD_SEPARATE: a separate pass owns each dq row and sums it in
 *                    registers, no atomics (bitwise identical run to run).
 *   FA_BWD_ORDERED:  the same atomic adds, made in ascending key-block order
 *                    for every 64-row dq tile through turn counters in the
 *                    workspace (bitwise identical run to run): the
 *                    semaphore-ordered reduction the page "FlashAttention-4"
 *                    names under "Limitations" for its deterministic mode.
 *   FA_BWD_ATOMIC_PAIRED: as FA_BWD_ATOMIC with half the atomic adds (the
 *                    restructured dQ of the page "FlashAttention-4", Key
 *                    Contributions item 3): key blocks 2p and 2p + 1 (128
 *                    keys each) of a kv head are paired, and for every query
 *                    tile both see the even block hands its partial dQ
 *                    tile to the odd one through the workspace, which adds
 *                    the sum.  The hand-over goes through the L2 of the XCD
 *                    both workgroups run on, or through memory when they run
 *                    on different XCDs (the same sum either way).
 */
#define FA_BWD_ATOMIC 0
#define FA_BWD_SEPARATE 1
#define FA_BWD_ORDERED 2
#define FA_BWD_ATOMIC_PAIRED 3

/*
 * Bytes of device workspace fa_bwd needs for this shape and dQ mode: the
 * per-row D_i = sum_c dO_ic O_ic and the base-2 LSE, two fp32 arrays
 * [B, Hq, N'] with N' = N rounded up to a multiple of 64, each rounded up to
 * 256 bytes; FA_BWD_ORDERED adds, right after them (at byte offset
 * fa_bwd_workspace_bytes(..., FA_BWD_SEPARATE)), a block of int32 counters:
 * 64 words, then 4 words per (batch, query head, 64 rows of N').  Word 1 of
 * that block counts the waits for a turn that gave up after about 2 s; it is
 * 0 after every call whose dq is bitwise reproducible (a non-zero count
 * leaves dq the correct sum, added in an unspecified order).
 * FA_BWD_ATOMIC_PAIRED adds, at the same offset, the pairing block: int32
 * words, 64 + 22 * B * Hkv * P of them with P = ceil(ceil(N / 128) / 2)
 * key-block pairs per kv head, rounded up to 256 bytes, then the hand-over
 * ring, 4 * 4 * B * Hkv * P tiles of 64 * d bytes.  Word 1 of the block
 * counts hand-over waits that gave up after about 2 s; a call that leaves it
 * non-zero has not added every partial to dq, and its dq must not be used
 * (it is 0 after every complete call).
 * Returns 0 for an invalid shape or mode.
 */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d, int deterministic);

/*
 * Backward attention.
 *   q, k, v   as in fa_fwd (read)
 *   o, lse    the forward's outputs for the same inputs (read)
 *   dout      bf16 [B, Hq, N, d], the gradient of the loss w.r.t. o (read)
 *   dq        fp32 [B, Hq,  N, d]  (written)
 *   dk, dv    fp32 [B, Hkv, N, d]  (written; summed over each group's heads)
 *   deterministic: the dQ mode, FA_BWD_ATOMIC (0), FA_BWD_SEPARATE (1),
 *     FA_BWD_ORDERED (2) or FA_BWD_ATOMIC_PAIRED (3), above; any other
 *     value is FA_ERR_SHAPE.  The reproducible modes repeat bit for bit on
 *     the same device and shape.
 *   workspace / workspace_bytes: device scratch of at least
 *     fa_bwd_workspace_bytes(...) bytes, 16-byte aligned, owned by the
 *     caller; its contents on entry are ignored.
 * Returns an fa_status.
 */
int fa_bwd(const void *q, const void *k, const void *v, const float *o, const float *lse,
           const void *dout, float *dq, float *dk, float *dv,
           int B, int Hq, int Hkv, int N, int d, float scale, int causal, int deterministic,
           void *workspace, size_t workspace_bytes, void *stream);

/*
 * fa_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The same kernels and results as fa_bwd
 * with the same dQ mode (the reproducible modes give the same bits); the
 * workspace fa_bwd would take lives instead in a static device array of the
 * library, FA_NOALLOC_MAX_WORKSPACE bytes on every device it runs on, held
 * until the process ends.  The call allocates nothing; its first call on a
 * device looks the array's address up (hipGetSymbolAddress).
 *   Limit: fa_bwd_workspace_bytes(B, Hq, Hkv, N, d, deterministic) must not
 *     exceed FA_NOALLOC_MAX_WORKSPACE (about 4 million rows B * Hq * N,
 *     e.g. B = 1, Hq = 32, N = 131072; in FA_BWD_ATOMIC_PAIRED the hand-over
 *     ring, 128 KiB per pair of 128-key blocks at d = 128, counts too, so
 *     that about 250 such pairs fit, e.g. B = 1, Hkv = 8, N = 4096);
 *     otherwise FA_ERR_WORKSPACE, before anything is enqueued.
 *   Every call on one device shares that device's array: calls that overlap
 *   in time on one device (different streams, or different host threads
 *   without ordering) race and give wrong results.  Calls ordered on one
 *   stream are safe; each call rewrites all of the array it uses.
 * Other arguments as in fa_bwd.  A failed address lookup is FA_ERR_HIP.
 * Returns an fa_status.
 */
#define FA_NOALLOC_MAX_WORKSPACE ((size_t)32 << 20)
int fa_bwd_noalloc(const void *q, const void *k, const void *v, const float *o,
                   const float *lse, const void *dout, float *dq, float *dk, float *dv,
                   int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                   int deterministic, void *stream);

/*
 * Backward of fa_fwd_window (same band; o and lse from fa_fwd_window with the
 * same window).  Arguments, workspace (fa_bwd_workspace_bytes) and modes as
 * in fa_bwd; window >= 1, otherwise FA_ERR_SHAPE.
 * Returns an fa_status.
 */
int fa_bwd_window(const void *q, const void *k, const void *v, const float *o, const float *lse,
                  const void *dout, float *dq, float *dk, float *dv,
                  int B, int Hq, int Hkv, int N, int d, float scale, int window,
                  int deterministic, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Forward with a linear position bias: every scaled score gets
 * slopes[h] * (j - i) added for query head h, query i and key j,
 *   S_ij = scale * q_i . k_j + slopes[h] * (j - i),
 * and O = softmax(S) v, LSE_i = ln sum_j exp(S_ij).  This is the additive
 * score modification of the FlexAttention kind that the page
 * "FlashAttention-4 Guide: Kernel Pipelining on Blackwell", section
 * "Production Deployment Guide", points to for custom masks and biases (the
 * pages give no formula; the ALiBi form, a fixed slope per head times the
 * signed key - query distance, is the reading stated here).
 *   slopes  fp32 [Hq], device memory, 4-byte aligned (read).  Non-finite
 *           slopes give non-finite outputs; values are not checked.
 * The bias is added in fp32 to the raw score q_i . k_j as
 * slopes[h] / scale * (j - i), so its rounding grows with |slopes[h]| * N / scale:
 * about 2^-24 of that, times scale * log2(e), enters the exponent.  It stays
 * far below the outputs' tolerance for ALiBi-sized slopes (<= 1) at the
 * sequence lengths tested here (N <= 8192).
 * causal as in fa_fwd; other arguments and outputs as in fa_fwd.  The
 * exponentials always run on the transcendental unit (FA_EXP2_POLY is
 * ignored); FA_RESCALE_TAU applies.  slopes == NULL is FA_ERR_NULL.
 * Returns an fa_status.
 */
int fa_fwd_alibi(const void *q, const void *k, const void *v, float *o, float *lse,
                 const float *slopes, int B, int Hq, int Hkv, int N, int d, float scale,
                 int causal, void *stream);

/*
 * Backward of fa_fwd_alibi (o and lse from fa_fwd_alibi with the same
 * slopes and causal flag); P is recomputed with the bias, the gradient
 * formulas are unchanged (the bias depends on neither q, k nor v).
 * Arguments, workspace (fa_bwd_workspace_bytes) and dQ modes as in fa_bwd;
 * slopes as in fa_fwd_alibi.
 * Returns an fa_status.
 */
int fa_bwd_alibi(const void *q, const void *k, const void *v, const float *o, const float *lse,
                 const void *dout, float *dq, float *dk, float *dv, const float *slopes,
                 int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                 int deterministic, void *workspace, size_t workspace_bytes, void *stream);

/* Static, human-readable name of a status code (never NULL). */
const char *fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
