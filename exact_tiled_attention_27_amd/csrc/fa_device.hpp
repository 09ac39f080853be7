// fa_device.hpp -- gfx950 device building blocks for the attention kernels.
//
// MFMA v_mfma_f32_32x32x16_bf16 (one wave of 64 lanes, lane l, half h = l/32):
//   A (32 x 16):  lane l holds A[l % 32][k-slots of half h]      (8 bf16)
//   B (16 x 32):  lane l holds B[k-slots of half h][l % 32]      (8 bf16)
//   C (32 x 32):  lane l holds C[8*(r/4) + 4*h + r%4][l % 32], r = 0..15
// A and B map (half, slot) to the contraction index identically, so any
// consistent assignment of physical contraction indices to (half, slot)
// computes the same product; the kernels use that freedom to feed a C result
// straight back as a B operand (the contraction runs over C's rows).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Hardware base-2 exponential (v_exp_f32): exp2(-inf) = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Pack 8 fp32 values into bf16 (round to nearest even).
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                              float a5, float a6, float a7)
{
    bf16x8 r;
    r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
    r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
    return r;
}

// Registers 8*j .. 8*j+7 of a 32x32 accumulator as a bf16 B operand.
__device__ __forceinline__ bf16x8 pack_half(const f32x16 &c, int j)
{
    return pack_bf16x8(c[8 * j + 0], c[8 * j + 1], c[8 * j + 2], c[8 * j + 3], c[8 * j + 4],
                       c[8 * j + 5], c[8 * j + 6], c[8 * j + 7]);
}

// acc + lo + hi for the two bf16 values packed in `pair` (bits 0-15 and
// 16-31): one v_dot2c_f32_bf16 against (1.0, 1.0), products exact.
__device__ __forceinline__ float sum_bf16_pair(uint32_t pair, float acc)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), ones, acc, false);
}

// LDS (address space 3) 16-byte reads at a byte offset.
__device__ __forceinline__ bf16x8 lds_read_bf16x8(const char *lds, uint32_t byte_off)
{
    return *reinterpret_cast<const bf16x8 *>(lds + byte_off);
}
__device__ __forceinline__ f32x4 lds_read_f32x4(const char *lds, uint32_t byte_off)
{
    return *reinterpret_cast<const f32x4 *>(lds + byte_off);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane j names 4 consecutive 16-bit values, row j of a 16 x 4 block M; lane i
// receives M[i/4 + 4u][i%4] for u = 0..3.  When lane j points at row
// (r0 + j/4), columns c0 + 4*(j%4) .. +3 of a row-major matrix, lane i receives
// column c0 + i of rows r0 .. r0+3: a 4 x 16 block transposed into registers.
__device__ __forceinline__ i16x4 lds_read_tr16(const char *lds, uint32_t byte_off)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(lds + byte_off));
}

// Two 4-element transposed reads as one 8-element bf16 MFMA operand.
__device__ __forceinline__ bf16x8 join_bf16x8(i16x4 lo, i16x4 hi)
{
    i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

// 16-byte global load with a zero fill when the row is out of range.
__device__ __forceinline__ u32x4 gload16(const void *base, size_t byte_off, bool ok)
{
    u32x4 z = {0u, 0u, 0u, 0u};
    return ok ? *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(base) + byte_off) : z;
}

// Make the compiler wait for the loads that produced `x` here.  Tile copies
// issued as inline assembly are invisible to its wait counting, so a load of
// its own still in flight at the first copy would later be waited for with a
// count that also drains those copies; kernels settle their own loads with
// this before the first copy.
template <typename T>
__device__ __forceinline__ void settle(const T &x)
{
    asm volatile("" ::"v"(x));
}

// Workgroup barrier that only hands off LDS: waits for this wave's LDS
// operations, not for its outstanding global loads, stores or atomics (a plain
// __syncthreads() also drains those, which would stall every loop iteration on
// the previous iteration's fire-and-forget atomics).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Reductions across the two 32-lane halves of a wave (lanes l and l ^ 32)
// with one v_permlane32_swap: afterwards lane l holds lanes 0-31's value in
// the first word and lanes 32-63's in the second, in both halves, so every
// lane computes the same bits.
// (The builtin exists only for the device target.)
__device__ __forceinline__ void halves_pair(float x, float &lo, float &hi)
{
#if defined(__HIP_DEVICE_COMPILE__)
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
#else
    lo = hi = x;
#endif
}
__device__ __forceinline__ float halves_max(float x)
{
    float lo, hi;
    halves_pair(x, lo, hi);
    return fmaxf(lo, hi);
}
__device__ __forceinline__ float halves_sum(float x)
{
    float lo, hi;
    halves_pair(x, lo, hi);
    return lo + hi;
}


// Round-robin dispatch puts workgroup i on XCD i % 8.  Map the hardware id to
// (head, tile) so each XCD works through whole heads: the workgroups that
// share one head's K/V run on the same XCD and share its L2.  With a causal
// mask the tiles of an XCD are issued longest first.  linear: the plain
// order instead (head-major, tile t of a head at id head * T + t), kept as a
// measurement switch for what the map above gains.
constexpr int kNumXcd = 8;
__device__ __forceinline__ void xcd_tile_map(int hw, int BH, int T, bool longest_first,
                                             bool linear, int &bh, int &t)
{
    if (linear) {
        bh = hw / T;
        t = hw % T;
    } else if (BH % kNumXcd == 0) {
        const int per = BH / kNumXcd;
        const int xcd = hw % kNumXcd, slot = hw / kNumXcd;
        if (longest_first) {
            t = T - 1 - slot / per;
            bh = xcd * per + slot % per;
        } else {
            bh = xcd * per + slot / T;
            t = slot % T;
        }
    } else if (longest_first) {
        t = T - 1 - hw / BH;
        bh = hw % BH;
    } else {
        bh = hw / T;
        t = hw % T;
    }
}

}  // namespace fa
