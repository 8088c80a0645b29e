// Device helpers shared by the attention kernels (gfx950): LDS layouts of
// 128-wide bf16 tiles, MFMA fragment reads, global -> LDS tile copies, and the
// lane-order fixes that turn a transposed 32 x 32 accumulator block into an
// MFMA operand or into 16-byte row stores.
//
// MFMA used throughout: v_mfma_f32_32x32x16_bf16.  Operand fragment: lane l
// holds 8 consecutive k (k = 8 (l / 32) + 0..7 of the 16-deep step) of row or
// column l % 32.  Accumulator: lane l holds column l % 32 and rows
// 8 (r / 4) + 4 (l / 32) + r % 4 for its 16 registers r.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace tps {
namespace attn {

constexpr int HD = 128;                       // head dim
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.69314718055994531f;

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;

// [rows][128] bf16 tiles, 256-byte rows of 16 chunks of 16 bytes; chunk c of
// row r sits at c ^ swz(r).  Layouts:
//   LAY_ROW:  swz = r % 16 -- 16 consecutive rows reading one logical chunk
//             (ds_read_b128) hit distinct banks;
//   LAY_COL:  rows r % 4 = 0,1,2,3 XOR with 0,6,10,12 -- the pattern the
//             transposing read uses without bank conflicts;
//   LAY_BOTH: swz = 4 (r % 4) + (r / 4) % 4 -- for tiles that are read both
//             ways: measured free of LDS bank conflicts on gfx950 for the row
//             reads (32 rows x one chunk pair, ds_read_b128) and for the
//             transposing column reads; the earlier 2 (r % 8) + (r / 8) % 2
//             was clean for rows but paid ~2 conflict cycles per column read.
enum : int { LAY_ROW = 0, LAY_COL = 1, LAY_BOTH = 2 };

template <int LAY>
__device__ __forceinline__ int swz(int r) {
  if constexpr (LAY == LAY_ROW) return r & 15;
  else if constexpr (LAY == LAY_COL) return (0xCA60 >> ((r & 3) * 4)) & 15;
  else return ((r & 3) << 2) | ((r >> 2) & 3);
}
template <int LAY>
__device__ __forceinline__ int toff(int r, int c) {
  return r * 256 + ((c ^ swz<LAY>(r)) << 4);
}

// Fragment with the tile's rows as MFMA rows/columns: row rb + lane % 32,
// k = columns 16 kk + 8 (lane / 32) .. +7.
template <int LAY>
__device__ __forceinline__ bf16x8 frag_rows(const TPS_LDS char* s, int rb, int kk) {
  const int lane = threadIdx.x & 63;
  const int r = rb + (lane & 31);
  return *reinterpret_cast<const TPS_LDS bf16x8*>(s + toff<LAY>(r, 2 * kk + (lane >> 5)));
}

// Fragment with the tile's columns as MFMA rows/columns: column cb + lane % 32,
// k = rows 16 kk + 8 (lane / 32) .. +7, through ds_read_b64_tr_b16 (within
// each 16-lane group, lane i gets element i % 4 of the 8-byte loads of lanes
// i/4, 4 + i/4, 8 + i/4, 12 + i/4).
template <int LAY>
__device__ __forceinline__ bf16x8 frag_cols(const TPS_LDS char* s, int cb, int kk) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 4, q = lane & 15;
  const int col = cb + 16 * (h & 1) + 4 * (q & 3);
  const int k0 = 16 * kk + 8 * (h >> 1) + (q >> 2);
  const int c = col >> 3, byte_in = (col & 7) * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TPS_LDS i16x4*)(s + toff<LAY>(k0, c) + byte_in));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TPS_LDS i16x4*)(s + toff<LAY>(k0 + 4, c) + byte_in));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Per-lane byte offsets of this wave's NB copy blocks of a [16 NB][128] tile
// (block NB w + j = rows 4 (NB w + j) .. +3; lane L writes bytes [16 L, 16 L + 16)
// of the block = row 4 B + L / 16, physical chunk L % 16).
template <int LAY, int NB>
__device__ __forceinline__ void tile_voffs(int64_t ld, uint32_t (&vo)[NB]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int row = 4 * (NB * wave + j) + (lane >> 4);
    const int c = (lane & 15) ^ swz<LAY>(row);
    vo[j] = (uint32_t)((row * ld + 8 * c) * 2);
  }
}

// Global -> LDS copies (buffer_load ... lds): lane i's 16 (4) bytes from byte offset voff of
// the buffer land at dst + 16 i (dst + 4 i); dst must be wave-uniform.  Written as inline
// assembly on purpose: for the builtin form the compiler makes every later transposing LDS
// read (ds_read_b64_tr_b16) wait for all outstanding copies, including the ones just issued
// for later tiles, which serialises the copy-ahead ring.  The kernels order copies and reads
// themselves (wait_vm on their own copies, then a workgroup barrier).
__device__ __forceinline__ void lds_copy16(const __amdgpu_buffer_rsrc_t& r, uint32_t voff, TPS_LDS char* dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void lds_copy4(const __amdgpu_buffer_rsrc_t& r, uint32_t voff, TPS_LDS char* dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "{m0}"(m0) : "memory");
}

template <int NB>
__device__ __forceinline__ void issue_tile(const __amdgpu_buffer_rsrc_t& r, const uint32_t (&vo)[NB], uint32_t off,
                                           TPS_LDS char* dst) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < NB; ++j) lds_copy16(r, vo[j] + off, dst + 1024 * (NB * wave + j));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t nrec) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nrec, 0x00020000);
}

// s_waitcnt vmcnt(VM): at most VM of this wave's vector memory operations (loads, LDS
// copies) still outstanding.  The 6-bit count is split over immediate bits 3:0 and 15:14;
// expcnt and lgkmcnt are left at their maxima (no wait).
template <int VM>
__device__ __forceinline__ void wait_vm() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
}

// B-operand fragment of k-step s from a 32 x 32 accumulator-shaped block
// packed to bf16 pairs (pk[2 q + w] = rows 8 q + 4 (l / 32) + 2 w, +1 of this
// lane's column): the step covers rows 16 s .. 16 s + 15 = quads 2 s, 2 s + 1;
// lanes < 32 hold rows +0..3 / +8..11, lanes >= 32 rows +4..7 / +12..15, and
// one v_permlane32_swap per register pair gives MFMA order (+0..7 | +8..15).
__device__ __forceinline__ bf16x8 pk_frag(const uint32_t (&pk)[8], int s) {
  const int q0 = 2 * s;
  uint32_t f[4];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const auto sw = __builtin_amdgcn_permlane32_swap(pk[2 * q0 + w], pk[2 * q0 + 2 + w], false, false);
    f[w] = sw[0];
    f[2 + w] = sw[1];
  }
  return __builtin_bit_cast(bf16x8, u32x4{f[0], f[1], f[2], f[3]});
}

// Row store of a transposed 32 x 128 result held as 4 accumulator blocks
// acc[db] (lane: row l % 32 of the result, columns 32 db + 8 (r / 4) +
// 4 (l / 32) + r % 4): values times `mul`, rounded to bf16; one swap per
// register pair gives each lane 8 consecutive columns for 16-byte stores.
// `row` points at the result row's first column; store = false skips the
// stores (the swaps still run on every lane).
__device__ __forceinline__ void store_rows_bf16(const f32x16 (&acc)[4], float mul, uint16_t* row, bool store) {
  const int lane = threadIdx.x & 63;
  uint16_t* p = row + 8 * (lane >> 5);
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    uint32_t pk[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) pk[q] = pack_bf2(acc[db][2 * q] * mul, acc[db][2 * q + 1] * mul);
#pragma unroll
    for (int pr = 0; pr < 2; ++pr)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const auto r = __builtin_amdgcn_permlane32_swap(pk[4 * pr + w], pk[4 * pr + 2 + w], false, false);
        pk[4 * pr + w] = r[0];
        pk[4 * pr + 2 + w] = r[1];
      }
    if (store) {
      *reinterpret_cast<u32x4*>(p + 32 * db) = u32x4{pk[0], pk[1], pk[2], pk[3]};
      *reinterpret_cast<u32x4*>(p + 32 * db + 16) = u32x4{pk[4], pk[5], pk[6], pk[7]};
    }
  }
}

// fp32 row store of the same transposed layout: lane writes 4 consecutive
// columns per register quad at row[32 db + 8 q + 4 (l / 32)].
__device__ __forceinline__ void store_rows_f32(const f32x16 (&acc)[4], float mul, float* row) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<f32x4*>(row + 32 * db + 8 * q + 4 * (lane >> 5)) =
          f32x4{acc[db][4 * q] * mul, acc[db][4 * q + 1] * mul, acc[db][4 * q + 2] * mul, acc[db][4 * q + 3] * mul};
}

}  // namespace attn
}  // namespace tps
