// Shared pieces of the gfx950 attention kernels: MFMA wrappers, the K-row
// order that makes every lane's P bytes 32 consecutive keys, LDS swizzles and
// the XCD-aware work order.
#pragma once
#include "vc_common.h"

namespace vc {

__device__ __forceinline__ int swz_k(int row) {
  return ((row >> 1) & 1) | (((row >> 2) & 1) << 1) | (((row >> 5) & 1) << 2);
}
__device__ __forceinline__ int swz_v(int row) { return (row >> 1) & 7; }

// Key (row of the 128-key tile) that MFMA row i of 32-key block m reads.
__device__ __forceinline__ int sigma(int m, int i) {
  return 64 * (m >> 1) + 32 * ((i >> 2) & 1) + 16 * (m & 1) + 4 * (i >> 3) + (i & 3);
}

__device__ __forceinline__ v16f mfma32(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i lds_op(const uint8_t* row_base, int chunk0, int swz) {
  const uint4 lo = *reinterpret_cast<const uint4*>(row_base + 16 * (chunk0 ^ swz));
  const uint4 hi = *reinterpret_cast<const uint4*>(row_base + 16 * ((chunk0 + 1) ^ swz));
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// Work item of this workgroup: items are (head, q-block) in head-major order,
// XCD x (= blockIdx % 8, the dispatch round robin) receives a contiguous range.
__device__ __forceinline__ int xcd_item(int id, int total) {
  const int x = id & 7, local = id >> 3;
  int start = 0;
  for (int y = 0; y < x; ++y) start += (total - y + 7) >> 3;
  return start + local;
}

// 16 bytes per lane from global memory straight into LDS: lane i of the wave
// writes lds_wave_base + 16*i (gfx950 global_load_lds_dwordx4).
__device__ __forceinline__ void dma16(const void* gsrc, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// Buffer-resource form of the same copy: the tile base stays in scalar
// registers (descriptor + soffset) and each lane adds a 32-bit offset, so no
// per-lane 64-bit address is kept live across a loop.  The descriptor's record
// count bounds the per-lane offset only (a lane offset at or past `bytes` reads
// zeros); the scalar offset is not checked, so callers keep it inside the record.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint8_t* lds_wave_base, uint32_t voff,
                                          uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                           (int)voff, (int)soff, 0, 0);
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

float score_scale_c0(float softmax_scale);

}  // namespace vc
