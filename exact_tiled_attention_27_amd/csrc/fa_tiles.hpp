// fa_tiles.hpp -- staging of bf16 [rows, D] tiles from HBM into LDS.
//
// Two LDS layouts, both read by MFMA operand loads of 16 bytes (8 bf16):
//
//  RowTile: row-major [ROWS][D].  The 16-byte chunk c of row r is stored at
//    chunk c ^ (r & 15) when D = 128 (c ^ (r & 7) when D = 64).  Sixteen
//    lanes reading the same chunk of 16 consecutive rows then hit 16 distinct
//    16-byte bank groups, which keeps 16-byte reads conflict-free whether the
//    LDS serves 8 or 16 lanes of them per clock.
//
//  VTile: row-major [ROWS][D] read with transposing 8-byte loads
//    (ds_read_b64_tr_b16): each 16-lane group reads 4 consecutive rows x 32
//    bytes, and the two groups of a 32-lane half read the same 4 rows 32 bytes
//    apart.  The chunk c of row r is stored at chunk c ^ (4 * (r & 3))
//    (D = 128): the 4 rows of one group land on 4 distinct 32-byte bank groups
//    and the two groups on disjoint ones, so the 32 lanes the LDS serves per
//    clock (256 bytes over 64 banks) never collide.
//
//  ColTile: transposed [D][ROWS] (one LDS row per head-dimension index d).
//    Sequence positions inside each group of 16 are stored either in natural
//    order or in key_pos16 order (the order in which a 32x32 accumulator
//    presents its rows to a B operand, so a C result can be contracted
//    against this tile without moving it).  Chunk j of LDS row d is stored
//    at chunk j ^ f(d), f(d) = (d & 7) ^ ((d >> 3) & 7): reads of one chunk
//    from 32 consecutive d rows and the transposing writes both spread over
//    the banks.
//
// Loads go global -> registers (16-byte loads, rows >= N read as zero) and
// registers -> LDS in a separate call, so the next tile's loads can be in
// flight while the current tile is computed.
#pragma once
#include "fa_device.hpp"

namespace fa {

__device__ __forceinline__ uint32_t row_tile_off(int row, int chunk, int D)
{
    return row * (D * 2) + ((chunk ^ (row & (D == 128 ? 15 : 7))) << 4);
}

__device__ __forceinline__ int vtile_swz(int row, int D)
{
    return D == 128 ? 4 * (row & 3) : 2 * (row & 3);
}

__device__ __forceinline__ uint32_t vtile_off(int row, int chunk, int D)
{
    return row * (D * 2) + ((chunk ^ vtile_swz(row, D)) << 4);
}

__device__ __forceinline__ int col_swz(int d) { return (d & 7) ^ ((d >> 3) & 7); }

template <int ROWS>
__device__ __forceinline__ uint32_t col_tile_off(int d, int chunk)
{
    return d * (ROWS * 2) + ((chunk ^ col_swz(d)) << 4);
}

__device__ __forceinline__ int row_swz(int row, int D) { return row & (D == 128 ? 15 : 7); }

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

// HBM -> LDS staging without registers (global_load_lds_dwordx4).  One wave
// instruction writes 1 KB of LDS: lane L's 16 bytes land at base + 16 L.  Each
// lane therefore fetches the logical chunk that the swizzled layout (RowTile
// or VTile) stores at that position: physical chunk p of row r holds logical
// chunk p ^ swz(r).  The tile's 1 KB blocks are split evenly over the waves;
// the per-lane byte offsets inside a tile are fixed, so a full tile costs no
// address arithmetic beyond one uniform base.  Completion is tracked by vmcnt.
template <int ROWS, int D, int THREADS, bool VSWZ>
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
            const int c = pc ^ (VSWZ ? vtile_swz(row, D) : row_swz(row, D));
            grow[i] = row;
            goff[i] = (row * D + c * 8) * 2;
        }
    }
    // All ROWS rows from row0 are < N.
    __device__ __forceinline__ void issue_full(const uint16_t *head, int row0, char *lds,
                                               int wave) const
    {
        const char *base = reinterpret_cast<const char *>(head) + (size_t)row0 * D * 2;
#pragma unroll
        for (int i = 0; i < PER_WAVE; i++)
            lds_dma16(base + goff[i], (lds_void_t *)(lds + (wave * PER_WAVE + i) * 1024));
    }
    // Tail tile: rows >= N re-read row N - 1 (finite data the caller masks).
    __device__ __forceinline__ void issue_tail(const uint16_t *head, int row0, int N, char *lds,
                                               int wave) const
    {
#pragma unroll
        for (int i = 0; i < PER_WAVE; i++) {
            const int n = min(row0 + grow[i], N - 1);
            const uint32_t within = goff[i] - grow[i] * D * 2;
            const char *src = reinterpret_cast<const char *>(head) + (size_t)n * D * 2 + within;
            lds_dma16(src, (lds_void_t *)(lds + (wave * PER_WAVE + i) * 1024));
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

template <int ROWS, int D, int THREADS, bool VSWZ = false>
struct RowTile {
    static constexpr int CPR = D / 8;  // 16-byte chunks per row
    static constexpr int TOTAL = ROWS * CPR;
    static constexpr int ITEMS = (TOTAL + THREADS - 1) / THREADS;
    static constexpr int BYTES = ROWS * D * 2;
    u32x4 x[ITEMS];

    __device__ __forceinline__ void load(const uint16_t *head, int row0, int N, int tid)
    {
#pragma unroll
        for (int i = 0; i < ITEMS; i++) {
            const int item = tid + i * THREADS;
            const int row = item / CPR, c = item % CPR;
            const int n = row0 + row;
            x[i] = gload16(head, ((size_t)n * D + c * 8) * 2, (TOTAL % THREADS == 0 || item < TOTAL) && n < N);
        }
    }
    // Rows row0 .. row0 + ROWS - 1 all < N: no guards, one uniform base.
    __device__ __forceinline__ void load_full(const uint16_t *head, int row0, int tid)
    {
        static_assert(TOTAL % THREADS == 0, "full loads need whole items per thread");
        const char *base = reinterpret_cast<const char *>(head) + (size_t)row0 * D * 2;
        const uint32_t toff = ((tid / CPR) * D + (tid % CPR) * 8) * 2;
#pragma unroll
        for (int i = 0; i < ITEMS; i++)
            x[i] = *reinterpret_cast<const u32x4 *>(base + toff + i * (THREADS / CPR) * D * 2);
    }
    __device__ __forceinline__ void store(char *lds, int tid) const
    {
#pragma unroll
        for (int i = 0; i < ITEMS; i++) {
            const int item = tid + i * THREADS;
            if (TOTAL % THREADS == 0 || item < TOTAL) {
                const int row = item / CPR, c = item % CPR;
                lds_write_u32x4(lds, VSWZ ? vtile_off(row, c, D) : row_tile_off(row, c, D), x[i]);
            }
        }
    }
};

template <int ROWS, int D, int THREADS, bool PERM>
struct ColTile {
    static constexpr int CPR = D / 8;
    static constexpr int TOTAL = (ROWS / 4) * CPR;  // items of 4 rows x 8 columns
    static constexpr int ITEMS = (TOTAL + THREADS - 1) / THREADS;
    static constexpr int BYTES = ROWS * D * 2;
    u32x4 x[ITEMS][4];

    __device__ __forceinline__ void load(const uint16_t *head, int row0, int N, int tid)
    {
#pragma unroll
        for (int i = 0; i < ITEMS; i++) {
            const int item = tid + i * THREADS;
            const int e = item % CPR, a = item / CPR;
            const bool live = TOTAL % THREADS == 0 || item < TOTAL;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int n = row0 + 4 * a + q;
                x[i][q] = gload16(head, ((size_t)n * D + e * 8) * 2, live && n < N);
            }
        }
    }
    // Transposed store: LDS row d, positions of rows 4a .. 4a+3.
    __device__ __forceinline__ void store(char *lds, int tid) const
    {
#pragma unroll
        for (int i = 0; i < ITEMS; i++) {
            const int item = tid + i * THREADS;
            if (TOTAL % THREADS == 0 || item < TOTAL) {
                const int e = item % CPR, a = item / CPR;
                const int kk = 4 * a;
                const int pos = PERM ? ((kk & ~15) | key_pos16(kk & 15)) : kk;
                const int chunk = pos >> 3, within = (pos & 7) * 2;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const uint32_t w0 = x[i][0][j], w1 = x[i][1][j], w2 = x[i][2][j],
                                   w3 = x[i][3][j];
                    // Column d = 8e + 2j takes the low halves, d + 1 the high halves.
                    const u32x2 lo = {(w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16)};
                    const u32x2 hi = {(w0 >> 16) | (w1 & 0xffff0000u),
                                      (w2 >> 16) | (w3 & 0xffff0000u)};
                    const int d0 = 8 * e + 2 * j;
                    lds_write_u32x2(lds, col_tile_off<ROWS>(d0, chunk) + within, lo);
                    lds_write_u32x2(lds, col_tile_off<ROWS>(d0 + 1, chunk) + within, hi);
                }
            }
        }
    }
    // The same registers stored row-major (RowTile layout).
    __device__ __forceinline__ void store_rows(char *lds, int tid) const
    {
#pragma unroll
        for (int i = 0; i < ITEMS; i++) {
            const int item = tid + i * THREADS;
            if (TOTAL % THREADS == 0 || item < TOTAL) {
                const int e = item % CPR, a = item / CPR;
#pragma unroll
                for (int q = 0; q < 4; q++)
                    lds_write_u32x4(lds, row_tile_off(4 * a + q, e, D), x[i][q]);
            }
        }
    }
};

}  // namespace fa
