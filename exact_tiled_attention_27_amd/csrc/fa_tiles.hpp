// fa_tiles.hpp -- LDS layout and HBM -> LDS staging of bf16 [rows, D] tiles.
//
// Every tile is stored row-major with an XOR swizzle of its 16-byte chunks
// (tile_swz), and reaches LDS through direct-to-LDS loads (DmaTile) with no
// staging registers.  Kernels read a tile two ways: 16-byte row reads give an
// MFMA operand whose contraction runs along the row (K for S^T = K Q^T, Q and
// dO for S and dP), and transposing 8-byte reads (tr_off) give an operand
// whose contraction runs down the columns (V^T, Q^T, dO^T, K^T).  One swizzle
// keeps both patterns free of bank conflicts.
#pragma once
#include "fa_device.hpp"

namespace fa {

// One swizzle for every row-major [rows][D] tile in LDS: the 16-byte chunk c
// of row r is stored at chunk c ^ tile_swz(r).  For D = 128 the swizzle swaps
// the two low 2-bit fields of the row index, (r & 3) << 2 | (r >> 2) & 3:
//  * 16-byte row reads (16 lanes, 16 consecutive rows, one chunk) hit 16
//    distinct 16-byte slots of the 256-byte bank window;
//  * transposing reads (32 lanes: 4 consecutive rows x two 32-byte column
//    groups) hit 8 distinct 32-byte slots.
// Both patterns are conflict-free on the 64-bank LDS.  For D = 64 (8 chunks
// per row) the 3-bit analogue keeps the transposing reads conflict-free.
__device__ __forceinline__ int tile_swz(int row, int D)
{
    return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : (((row & 3) << 1) | ((row >> 2) & 1));
}

__device__ __forceinline__ uint32_t tile_off(int row, int chunk, int D)
{
    return row * (D * 2) + ((chunk ^ tile_swz(row, D)) << 4);
}

// Byte offset of this lane's 8-byte transposing read (ds_read_b64_tr_b16) of
// rows row0 + r16/4 (r16 = lane % 16) and columns c0 + 4 (r16 % 4) .. +3 of a
// row-major tile; c0 is a multiple of 16.  Lane i of each 16-lane group then
// receives column c0 + i of rows row0 .. row0 + 3.
__device__ __forceinline__ uint32_t tr_off(int row0, int c0, int lane, int D)
{
    const int r16 = lane & 15;
    const int row = row0 + (r16 >> 2);
    const int col = c0 + 4 * (r16 & 3);
    return tile_off(row, col >> 3, D) + (col & 7) * 2;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// 16-byte global -> LDS copy (global_load_lds_dwordx4; LDS base wave-uniform).
// The builtin exists only for the device target; the host pass, which only
// needs the kernels' launch stubs, must not see it (when it does, clang drops
// some template instantiations of the kernels from the host object).
__device__ __forceinline__ void lds_dma16(const void *src, lds_void_t *dst)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
#else
    (void)src;
    (void)dst;
#endif
}

// Raw buffer resource over one head's [N][D] bf16 rows: base address, stride
// 0, size in bytes, 32-bit data format.  It sits in scalar registers, so a
// buffer copy into LDS takes a per-lane 32-bit offset plus a scalar row
// offset and needs no per-copy address arithmetic.
struct BufRsrc {
    int r __attribute__((ext_vector_type(4)));
};

__device__ __forceinline__ BufRsrc make_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    BufRsrc x;
    x.r[0] = (int)(uint32_t)a;
    x.r[1] = (int)((a >> 32) & 0xffffu);  // stride 0, no swizzle
    x.r[2] = (int)bytes;
    x.r[3] = 0x00020000;
    return x;
}

// 16-byte buffer -> LDS copy (buffer_load_dwordx4 ... lds; LDS base in M0).
// Issued as inline assembly so that the compiler does not wait for it before
// unrelated LDS reads; completion is awaited explicitly (dma_barrier).  The
// s_nop covers the M0-write -> LDS-DMA hazard.
__device__ __forceinline__ void lds_dma16_buf(const BufRsrc &rs, uint32_t voff, uint32_t soff,
                                              lds_void_t *dst)
{
    const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>(dst);
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "{m0}"(m0), "v"(voff), "s"(rs.r), "s"(soff) : "memory");
}

// The same copy without a memory clobber: for copies placed between matrix
// products (the step barriers, which carry the clobber, order them against
// every LDS access of the slot they fill).
__device__ __forceinline__ void lds_dma16_buf_nc(const BufRsrc &rs, uint32_t voff, uint32_t soff,
                                                 lds_void_t *dst)
{
    const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>(dst);
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "{m0}"(m0), "v"(voff), "s"(rs.r), "s"(soff));
}

// HBM -> LDS staging of a [ROWS][D] bf16 tile without registers
// (global_load_lds_dwordx4).  One wave instruction writes 1 KB of LDS: lane
// L's 16 bytes land at base + 16 L, so each lane fetches the logical chunk the
// swizzled layout stores at that position (physical chunk p of row r holds
// logical chunk p ^ tile_swz(r)).  The tile's 1 KB blocks are split evenly
// over the waves; per-lane offsets are fixed, so a full tile needs one
// uniform base per call.  Completion is tracked by vmcnt.
template <int ROWS, int D, int THREADS>
struct DmaTile {
    static constexpr int CPR = D / 8;                // 16-byte chunks per row
    static constexpr int BLOCKS = ROWS * CPR / 64;   // 1 KB blocks in the tile
    static constexpr int WAVES = THREADS / 64;
    static constexpr int PER_WAVE = BLOCKS / WAVES;
    static constexpr int BYTES = ROWS * D * 2;
    static_assert(BLOCKS % WAVES == 0, "tile must split evenly over the waves");
    uint32_t goff[PER_WAVE];  // byte offset of this lane's source chunk inside the tile
    int grow[PER_WAVE];       // tile row this lane fills for each block

    __device__ __forceinline__ void init(int wave, int lane)
    {
#pragma unroll
        for (int i = 0; i < PER_WAVE; i++) {
            const int pos = (wave * PER_WAVE + i) * 64 + lane;
            const int row = pos / CPR, pc = pos % CPR;
            const int c = pc ^ tile_swz(row, D);
            grow[i] = row;
            goff[i] = (row * D + c * 8) * 2;
        }
    }
    // Rows row0 .. row0 + ROWS - 1 of `head` (rows >= N re-read row N - 1:
    // finite data the caller masks).
    __device__ __forceinline__ void issue(const uint16_t *head, int row0, int N, char *lds,
                                          int wave) const
    {
        if (row0 + ROWS <= N) {
            const char *base = reinterpret_cast<const char *>(head) + (size_t)row0 * D * 2;
#pragma unroll
            for (int i = 0; i < PER_WAVE; i++)
                lds_dma16(base + goff[i], (lds_void_t *)(lds + (wave * PER_WAVE + i) * 1024));
        } else {
#pragma unroll
            for (int i = 0; i < PER_WAVE; i++) {
                const int n = min(row0 + grow[i], N - 1);
                const uint32_t within = goff[i] - grow[i] * D * 2;
                const char *src = reinterpret_cast<const char *>(head) + (size_t)n * D * 2 + within;
                lds_dma16(src, (lds_void_t *)(lds + (wave * PER_WAVE + i) * 1024));
            }
        }
    }
    // Block i of a full tile (rows row0 .. row0 + ROWS - 1 all < N), alone.
    __device__ __forceinline__ void issue_block(const BufRsrc &rs, int row0, char *lds, int wave,
                                                int i) const
    {
        lds_dma16_buf_nc(rs, goff[i], (uint32_t)row0 * (D * 2),
                         (lds_void_t *)(lds + (wave * PER_WAVE + i) * 1024));
    }
    // The same copy from a buffer resource over the head's rows (every
    // offset stays below N * D * 2 bytes).
    __device__ __forceinline__ void issue(const BufRsrc &rs, int row0, int N, char *lds,
                                          int wave) const
    {
        if (row0 + ROWS <= N) {
            const uint32_t soff = (uint32_t)row0 * (D * 2);
#pragma unroll
            for (int i = 0; i < PER_WAVE; i++)
                lds_dma16_buf(rs, goff[i], soff, (lds_void_t *)(lds + (wave * PER_WAVE + i) * 1024));
        } else {
#pragma unroll
            for (int i = 0; i < PER_WAVE; i++) {
                const int n = min(row0 + grow[i], N - 1);
                const uint32_t voff = (uint32_t)n * (D * 2) + (goff[i] - grow[i] * D * 2);
                lds_dma16_buf(rs, voff, 0u, (lds_void_t *)(lds + (wave * PER_WAVE + i) * 1024));
            }
        }
    }
};

// Wait for this wave's outstanding global loads (including loads into LDS)
// and LDS operations, then meet the workgroup: afterwards every wave's
// direct-to-LDS tile is complete and visible.
__device__ __forceinline__ void dma_barrier()
{
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace fa
