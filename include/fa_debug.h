/*
 * fa_debug.h -- extra C ABI of the debug build libfa_debug.so.
 *
 * libfa_debug.so is the same library as libfa.so (every entry point of
 * fa.h, same kernels) built with event counters in the forward kernels.  It
 * exists to measure what the method's choices do on a real workload: how
 * often the conditional rescale of the running maximum is taken (page
 * "FlashAttention-4", section "Key Contributions", item 2: the accumulator is
 * only renormalised when the maximum grows by more than log2(256) = 8), and
 * how many key tiles the causal and sliding-window maps skip or mask.  The
 * counters add atomics to the kernels, so timings of this build are not
 * representative; libfa.so has none of them.
 */
#ifndef FA_DEBUG_H
#define FA_DEBUG_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Counter indices (n values are copied; missing ones stay untouched):
 *   0  rescale decisions: (query row, key tile) pairs of the tiles a row's
 *      workgroup walks after the row's first tile with a valid key (that
 *      one always sets the reference; later tiles whose keys are all masked
 *      for the row count as decisions that never move it)
 *   1  of those, the pairs whose tile maximum exceeded the reference by more
 *      than the threshold, so the row's reference moved
 *   2  waves that took the rescale branch (some row of the wave moved)
 *   3  key tiles walked (64 keys each), summed over workgroups
 *   4  of those, tiles that took the masked path (causal diagonal, sequence
 *      tail, sliding-window edge)
 *   5  workgroups launched
 * The counters sum over every forward call since the last read (fa_fwd,
 * fa_fwd_window, fa_fwd_splitkv, fa_fwd_alibi; not the backward) on the
 * current device.  Copies min(n, 6) counters into host memory `counters`,
 * then clears them; synchronises the device.  counters == NULL or n < 1 is
 * FA_ERR_NULL; a HIP error is FA_ERR_HIP.
 */
int fa_debug_counters(unsigned long long *counters, int n);

/*
 * The dQ atomics of the backward's atomic modes, alone: the device's rate
 * for them is what bounds those modes (every such fp32 add is executed at
 * the memory side, not in an XCD's L2).  `blocks` workgroups of 256 threads
 * each add `tiles` tiles of 64 x 128 fp32 values 1.0 into tile slot
 * (7 w + 13 i) % n_slots of buf (w the workgroup, i the tile; each slot
 * 64 * 128 floats), with the lane pattern of the dK/dV kernel's dQ adds.
 * buf: fp32 device memory of at least n_slots * 64 * 128 floats, 16-byte
 * aligned.  Enqueued on `stream`; FA_ERR_NULL / FA_ERR_SHAPE / FA_ERR_ALIGN
 * for bad arguments, FA_ERR_HIP for a launch error.
 */
int fa_debug_atomic_tiles(float *buf, int n_slots, int tiles, int blocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_DEBUG_H */
