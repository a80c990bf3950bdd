// Test hook: single gfx950 instructions on caller data.  The attention and
// preprocessing kernels rest on a few facts about these instructions (the FP8
// matrix instructions' accumulation, the rounding and range of the two byte
// conversions, the accuracy of the hardware exp2); this entry point runs each
// instruction alone so that tests can record those facts against exact
// arithmetic on the host.  Three plain HBM streams (read only, copy, two reads
// per write) measure the bandwidth the memory-bound passes can reach; three rate
// kernels measure the FP8 matrix-instruction throughput, how fast one or two
// wavefronts per SIMD issue vector instructions, and how fast a CU issues the
// global -> LDS copies that stage the attention tiles.
#include "attn_common.h"

namespace vc {

// V_CVT_PK_FP8_F32 without the clamp the encoders apply (what = 0)
__global__ void probe_cvt_fp8(const float* in, uint8_t* out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(in[i], 0.0f, 0u, false) & 0xFFu);
}

// V_CVT_PK_U8_F32 (what = 1)
__global__ void probe_cvt_u8(const float* in, uint8_t* out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (uint8_t)(__builtin_amdgcn_cvt_pk_u8_f32(in[i], 0, 0u) & 0xFFu);
}

// V_EXP_F32 (what = 2)
__global__ void probe_exp2(const float* in, float* out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = __builtin_amdgcn_exp2f(in[i]);
}

// One wavefront per tile: D = A . B^T + C with V_MFMA_F32_32X32X64_F8F6F4 (what
// = 3, M = N = 32, K = 64) or V_MFMA_F32_16X16X128_F8F6F4 (what = 4, M = N = 16,
// K = 128), E4M3 operands.  Tile layout in `in`: A [M][K] bytes, B [N][K]
// bytes, C [M][N] fp32; in `out`: D [M][N] fp32.  Lane l holds row (or column)
// l % M and the K-slice 32 (l / M) .. 32 (l / M) + 31 of both operands.
template <int M>
__global__ void __launch_bounds__(64) probe_mfma(const uint8_t* in, float* out, int tiles) {
  constexpr int K = 2048 / M;
  constexpr int tile_bytes = 2 * M * K + 4 * M * M;
  const int tile = blockIdx.x, l = threadIdx.x;
  if (tile >= tiles) return;
  const uint8_t* A = in + (long long)tile * tile_bytes;
  const uint8_t* B = A + M * K;
  const float* C = reinterpret_cast<const float*>(B + M * K);
  float* D = out + (long long)tile * M * M;
  const int r = l % M, kg = l / M;
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = *reinterpret_cast<const int*>(A + r * K + 32 * kg + 4 * i);
    b[i] = *reinterpret_cast<const int*>(B + r * K + 32 * kg + 4 * i);
  }
  if constexpr (M == 32) {
    v16f c;
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = C[(8 * (i >> 2) + 4 * kg + (i & 3)) * M + r];
    const v16f d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) D[(8 * (i >> 2) + 4 * kg + (i & 3)) * M + r] = d[i];
  } else {
    v4f c;
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = C[(4 * kg + i) * M + r];
    const v4f d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) D[(4 * kg + i) * M + r] = d[i];
  }
}

// HBM streams over n 16-byte words, 2048 workgroups of 256 threads striding the
// array: read only (what = 5: in [n], one XOR per thread to out [2048 * 256]),
// copy (what = 6: in [n] -> out [n]), two reads per write (what = 7: out[i] =
// in[i] ^ in[i + n], in [2n], out [n]).
constexpr int kStreamGrid = 2048;
__global__ void __launch_bounds__(256) probe_read(const uint4* __restrict__ a, long long n, uint32_t* __restrict__ out) {
  uint32_t x = 0u;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const uint4 v = a[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[blockIdx.x * 256 + threadIdx.x] = x;
}
__global__ void __launch_bounds__(256) probe_copy(const uint4* __restrict__ a, uint4* __restrict__ b, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) b[i] = a[i];
}
__global__ void __launch_bounds__(256) probe_read2_write1(const uint4* __restrict__ a, uint4* __restrict__ b,
                                                          long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const uint4 u = a[i], v = a[i + n];
    b[i] = make_uint4(u.x ^ v.x, u.y ^ v.y, u.z ^ v.z, u.w ^ v.w);
  }
}

// FP8 MFMA throughput (what = 8): n workgroups of 256 threads (one wavefront per
// SIMD), each wavefront kMfmaIters iterations of four independent
// V_MFMA_F32_32X32X64_F8F6F4 on register operands taken from `in` (E4M3 bytes,
// 2 KiB); out [n * 256] receives each thread's accumulator sum, so nothing is
// optimised away.  131072 FLOP per instruction.
constexpr int kMfmaIters = 2048;
__global__ void __launch_bounds__(256) probe_mfma_rate(const uint8_t* __restrict__ in, float* __restrict__ out) {
  const int tid = threadIdx.x;
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = reinterpret_cast<const int*>(in)[(tid * 8 + i) & 511];
    b[i] = reinterpret_cast<const int*>(in)[(tid * 5 + i + 7) & 511];
  }
  v16f acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  for (int it = 0; it < kMfmaIters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 0, 0, 0, 0, 0);
  }
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[j][r];
  out[blockIdx.x * 256 + tid] = sum;
}

// VALU issue rate (what = 9): n workgroups of 512 threads, one per CU (the
// LDS array keeps a second one off), wavefront w on SIMD w % 4.  in[0] selects
// the instruction (0: V_FMA_F32, 1: V_EXP_F32 of -|x|), in[1] the number of
// wavefronts that run it (4: one per SIMD, 8: two); each runs kValuIters
// iterations of eight independent chains.  out [n * 8][2] int64: per wavefront
// the s_memtime ticks of its loop (0 for idle wavefronts) and the bits of its
// lane-0 chain sum (so the chains are not optimised away).
constexpr int kValuIters = 4096;
__global__ void __launch_bounds__(512) probe_valu_rate(const int* __restrict__ cfg, long long* __restrict__ out) {
  __shared__ float pad[24576];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int mode = cfg[0], active = cfg[1];
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 0.01f * (float)((tid + 3 * i) & 63) - 0.3f;
  pad[tid] = x[0];
  __syncthreads();
  long long t0 = 0, t1 = 0;
  if (wave < active) {
    t0 = __builtin_amdgcn_s_memtime();
    if (mode == 0) {
      for (int it = 0; it < kValuIters; ++it)
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(x[i], 0.999f, -0.25f);
    } else {
      for (int it = 0; it < kValuIters; ++it)
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(-__builtin_fabsf(x[i]));
    }
    t1 = __builtin_amdgcn_s_memtime();
  }
  float sum = pad[(tid + 64) & 511];
#pragma unroll
  for (int i = 0; i < 8; ++i) sum += x[i];
  if ((tid & 63) == 0) {
    out[2 * (blockIdx.x * 8 + wave)] = t1 - t0;
    out[2 * (blockIdx.x * 8 + wave) + 1] = (long long)__float_as_uint(sum);
  }
}

typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

// Global -> LDS copy rate (what = 10): n workgroups of 512 threads, one per CU
// (the LDS array keeps a second one off).  `in` holds i32 {mode, iterations} in
// its first 256 bytes and an 8 KiB source after them, which every wavefront
// reads again and again (it stays in the caches).  Each iteration a wavefront
// issues eight 64-lane loads through a buffer resource and then waits for them:
// mode 0 `buffer_load_dwordx4 ... lds` (16 bytes per lane into LDS), mode 1
// `buffer_load_dword ... lds` (4 bytes per lane into LDS), mode 2
// `buffer_load_dwordx4` into registers (XORed into a checksum).  out [n * 8][2]
// int64: per wavefront the s_memtime ticks of its loop and a checksum that keeps
// the loads alive.
__global__ void __launch_bounds__(512) probe_lds_copy(const uint8_t* __restrict__ in, long long* __restrict__ out) {
  __shared__ __align__(16) uint8_t buf[98304];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int mode = reinterpret_cast<const int*>(in)[0];
  const int iters = reinterpret_cast<const int*>(in)[1];
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(in + 256, 8192u);   // lane offsets below stay under 8 KiB
  uint8_t* dst = buf + 8192 * wave;                               // eight 1 KiB slots per wavefront
  for (int i = tid; i < 98304 / 16; i += 512) reinterpret_cast<uint4*>(buf)[i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  uint32_t acc = 0u;
  const long long t0 = __builtin_amdgcn_s_memtime();
  if (mode == 0) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) dma16_buf(rs, dst + 1024 * j, (uint32_t)(16 * lane + 1024 * j), 0u);
      wait_dma();
    }
  } else if (mode == 1) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 1024 * j), 4,
                                                 4 * lane + 256 * j, 0, 0, 0);
      wait_dma();
    }
  } else {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // the lane offset moves with the iteration (inside the same 1 KiB), so the
        // loads cannot be hoisted out of the loop
        const uint32_t off = (uint32_t)(1024 * j + ((16 * lane) ^ (16 * (it & 63))));
        const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0u, 0);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
      }
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  __syncthreads();
  acc ^= reinterpret_cast<const uint32_t*>(buf)[(tid * 37) & 16383];   // inside the copied 64 KiB
  if (lane == 0) {
    out[2 * (blockIdx.x * 8 + wave)] = t1 - t0;
    out[2 * (blockIdx.x * 8 + wave) + 1] = (long long)acc;
  }
}

}  // namespace vc

using namespace vc;

extern "C" int vc_device_probe(int what, const void* in, void* out, int n, void* stream) {
  if (!in || !out || n < 1) return VC_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  switch (what) {
    case 0: hipLaunchKernelGGL(probe_cvt_fp8, grid, block, 0, st, (const float*)in, (uint8_t*)out, n); break;
    case 1: hipLaunchKernelGGL(probe_cvt_u8, grid, block, 0, st, (const float*)in, (uint8_t*)out, n); break;
    case 2: hipLaunchKernelGGL(probe_exp2, grid, block, 0, st, (const float*)in, (float*)out, n); break;
    case 3: hipLaunchKernelGGL(probe_mfma<32>, dim3((unsigned)n), dim3(64), 0, st, (const uint8_t*)in, (float*)out, n); break;
    case 4: hipLaunchKernelGGL(probe_mfma<16>, dim3((unsigned)n), dim3(64), 0, st, (const uint8_t*)in, (float*)out, n); break;
    case 5: hipLaunchKernelGGL(probe_read, dim3(kStreamGrid), block, 0, st, (const uint4*)in, (long long)n, (uint32_t*)out); break;
    case 6: hipLaunchKernelGGL(probe_copy, dim3(kStreamGrid), block, 0, st, (const uint4*)in, (uint4*)out, (long long)n); break;
    case 7:
      hipLaunchKernelGGL(probe_read2_write1, dim3(kStreamGrid), block, 0, st, (const uint4*)in, (uint4*)out, (long long)n);
      break;
    case 8: hipLaunchKernelGGL(probe_mfma_rate, dim3((unsigned)n), block, 0, st, (const uint8_t*)in, (float*)out); break;
    case 9:
      hipLaunchKernelGGL(probe_valu_rate, dim3((unsigned)n), dim3(512), 0, st, (const int*)in, (long long*)out);
      break;
    case 10:
      hipLaunchKernelGGL(probe_lds_copy, dim3((unsigned)n), dim3(512), 0, st, (const uint8_t*)in, (long long*)out);
      break;
    default: return VC_ERR_UNSUPPORTED;
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? VC_OK : vc_set_hip_error((int)e);
}
