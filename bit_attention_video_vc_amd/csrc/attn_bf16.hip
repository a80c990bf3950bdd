// Comparator: standard non-causal flash attention in bf16 on gfx950.
//
// The pages quote every attention speed-up against BF16 FlashAttention-4
// (insight article, section "A Faster Kernel Does Not Automatically Mean
// Faster Generation"; paper digest, results table).  This kernel is the in-repo
// stand-in on MI355X: bf16 V_MFMA_F32_32X32X16_BF16 for Q.K^T and P.V, online
// softmax with fp32 exp2, P rounded to bf16 (round to nearest even), row sums of
// the rounded P accumulated in fp32 by a bf16 MFMA.
//
// Same organisation as the FP8 kernel: S^T = K.Q^T so each lane holds one
// query's scores and the bf16 P values are already in the B-operand layout of
// O^T = V^T.P^T.  A first kernel writes V transposed per 128-key block into the
// caller's workspace (one HBM pass); the attention kernel then streams K and V^T
// tiles global -> LDS directly through buffer resources, double buffered in
// 128 KiB of static LDS, 8 wavefronts (256 queries) per workgroup so that two
// wavefronts share each SIMD.  Operand reads address the LDS through per-lane
// registers plus constants that fit the instruction's 16-bit offset, so no
// address arithmetic sits beside the MFMAs.
#include <type_traits>

#include "attn_common.h"

namespace vc {

constexpr int kB16Threads = 512;
constexpr int kRowB = kD * 2;            // bytes per bf16 row (256)
constexpr int kTileB = kBlock * kRowB;   // bytes per bf16 tile (32 KiB)

struct B16Args {
  const uint16_t* q; const uint16_t* k; const uint16_t* vt;
  float* out;
  int N, nb, nqb, BH;
  float c0;
};

__device__ __forceinline__ int swz_kb(int row) {
  return (row & 3) | (((row >> 2) & 1) << 2) | (((row >> 5) & 1) << 3);
}

__device__ __forceinline__ v16f mfma_bf16(const v8bf& a, const v8bf& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf as_bf(uint4 u) {
  v8bf r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

// V [BH][N][128] -> V^T per block: vt[BH][nb][128 ch][128 keys], zero past N.
__global__ void __launch_bounds__(256) transpose_v_bf16(const uint16_t* __restrict__ V, int N, int nb,
                                                        uint16_t* __restrict__ vt) {
  __shared__ __align__(16) uint16_t tile[kBlock * (kD + 8)];   // padded rows
  const int t = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int n = min(kBlock, N - t * kBlock);
  for (int q = tid; q < kBlock * 16; q += 256) {
    const int r = q >> 4, c = q & 15;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < n) v = *reinterpret_cast<const uint4*>(V + ((long long)bh * N + t * kBlock + r) * kD + 8 * c);
    *reinterpret_cast<uint4*>(&tile[r * (kD + 8) + 8 * c]) = v;
  }
  __syncthreads();
  uint16_t* dst = vt + ((long long)bh * nb + t) * kBlock * kD;
  for (int q = tid; q < kD * 16; q += 256) {
    const int ch = q & (kD - 1), kc = q >> 7;   // channel, chunk of 8 keys
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tile[(8 * kc + 2 * e) * (kD + 8) + ch] |
             ((uint32_t)tile[(8 * kc + 2 * e + 1) * (kD + 8) + ch] << 16);
    *reinterpret_cast<uint4*>(dst + ch * kBlock + 8 * kc) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// 32-bit LDS address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(size_t)(const lds_u8*)(p);
}
// 16 bytes from LDS address `addr` (a register base plus a constant that fits
// the instruction's 16-bit offset)
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 lds_read16(uint32_t addr) {
  const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>((size_t)addr);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__global__ void __launch_bounds__(kB16Threads, 1) attn_bf16_kernel(B16Args a) {
  __shared__ __align__(16) uint8_t Kt[2][kTileB];   // [128 keys][256 B], swizzled chunks
  __shared__ __align__(16) uint8_t Vt[2][kTileB];   // [128 ch][256 B], swizzled chunks

  const int item = xcd_item(blockIdx.x, a.nqb * a.BH);
  const int bh = item / a.nqb, qb = item % a.nqb;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: copy destinations stay scalar
  const int g = lane >> 5, col = lane & 31;
  const int N = a.N, nb = a.nb;

  const int qrow = qb * 256 + wave * 32 + col;
  v8bf qop[8];
  {
    const uint16_t* qp = a.q + ((long long)bh * N + min(qrow, N - 1)) * kD;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint4 u = *reinterpret_cast<const uint4*>(qp + 16 * j + 8 * g);
      if (qrow >= N) u = make_uint4(0, 0, 0, 0);
      qop[j] = as_bf(u);
    }
  }
  // copies through buffer resources: K rows past N (lane offsets past the
  // head's N rows) read as zeros; V^T tiles are padded, their tile offset is scalar
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k + (long long)bh * N * kD, (uint32_t)N * kRowB);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.vt + (long long)bh * nb * kBlock * kD, (uint32_t)nb * kTileB);

  // DMA: instruction j (32 per operand per tile, 4 per wave) fills LDS bytes
  // [1024j, 1024j+1024) = rows 4j..4j+3; lane i writes row 4j + i/16 at chunk
  // position i%16.
  uint32_t dkoff[4], dvoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = 8 * i + wave;
    const int row = 4 * j + (lane >> 4), pos = lane & 15;
    dkoff[i] = (uint32_t)(row * kRowB + 16 * (pos ^ swz_kb(row)));
    dvoff[i] = (uint32_t)(row * kRowB + 16 * (pos ^ (row & 15)));
  }
  auto load_tile = [&](int t, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 8 * i + wave;
      dma16_buf(krs, Kt[buf] + 1024 * j, (uint32_t)t * kTileB + dkoff[i], 0u);   // rows past N: zeros, masked later
      dma16_buf(vrs, Vt[buf] + 1024 * j, dvoff[i], (uint32_t)t * kTileB);
    }
  };
  // LDS operand addresses (rows sigma(m, col) share the K swizzle, channels
  // 32*cb + col share the V^T swizzle)
  // per-lane LDS addresses of the operand reads (K tile 0 and V^T tile 0),
  // kept opaque so that every read is a register plus an in-range constant
  // (buffer, 32-key block, channel block): the V^T tiles lie above 64 KiB
  uint32_t lk[8], lv[8];
  {
    const int kr = sigma(0, col), ksw = swz_kb(kr), vsw = col & 15;
#pragma unroll
    for (int j = 0; j < 8; ++j) lk[j] = lds_addr(Kt[0]) + (uint32_t)(kr * kRowB + 16 * ((2 * j + g) ^ ksw));
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int chunk = 8 * (m >> 1) + 4 * g + 2 * (m & 1) + s2;
        lv[2 * m + s2] = lds_addr(Vt[0]) + (uint32_t)(col * kRowB + 16 * (chunk ^ vsw));
      }
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(lk[j]), "+v"(lv[j]));
  }

  load_tile(0, 0);
  wait_dma();
  __syncthreads();

  v16f o[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[cb][r] = 0.0f;
  float mx = -__builtin_inff(), l = 0.0f;
  // the row sums of the rounded P (the values the P.V product takes) come from
  // a 16x16x32 bf16 MFMA per 16-key chunk against a lane-parity ones pattern: the
  // 16x16x32 operand layout reads the chunk's registers as four 8-key slices
  // of columns l % 16, and the pattern keeps, in output row i, the slices of
  // query (i / 4) % 2 * 16 + column, so that lane l ends with query l % 32's sum
  v8bf ones;
  {
    const bool on = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1);
    ones = as_bf(on ? make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u) : make_uint4(0, 0, 0, 0));
  }

  auto step = [&](const int t, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    if (t + 1 < nb) load_tile(t + 1, buf ^ 1);

    v16f s[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[m][r] = 0.0f;
      const uint32_t kb = (uint32_t)(buf * kTileB + kRowB * (64 * (m >> 1) + 16 * (m & 1)));
#pragma unroll
      for (int j = 0; j < 8; ++j) s[m] = mfma_bf16(as_bf(lds_read16(lk[j] + kb)), qop[j], s[m]);
    }
    if ((t + 1) * kBlock > N) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 64 * (m >> 1) + 32 * g + 16 * (m & 1) + r;
          if (t * kBlock + key >= N) s[m][r] = -__builtin_inff();
        }
    }
    float M = s[0][0];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) M = fmaxf(M, s[m][r]);
    M = fmaxf(M, __shfl_xor(M, 32));
    const float mx_new = fmaxf(mx, M * a.c0);
    const float alpha = __builtin_amdgcn_exp2f(mx - mx_new);
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[cb][r] *= alpha;
    }
    l *= alpha;
    mx = mx_new;
    const float nmx = -mx_new;

    v4f rs = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        typedef float v2f __attribute__((ext_vector_type(2)));
        typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
        uint32_t pw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v2f p;
          p.x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[m][8 * s2 + 2 * e], a.c0, nmx));
          p.y = __builtin_amdgcn_exp2f(__builtin_fmaf(s[m][8 * s2 + 2 * e + 1], a.c0, nmx));
          const v2bf pb = __builtin_convertvector(p, v2bf);   // round to nearest even
          pw[e] = __builtin_bit_cast(uint32_t, pb);
        }
        const v8bf pop = as_bf(make_uint4(pw[0], pw[1], pw[2], pw[3]));
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const uint4 vv = lds_read16(lv[2 * m + s2] + (uint32_t)(buf * kTileB + kRowB * 32 * cb));
          o[cb] = mfma_bf16(as_bf(vv), pop, o[cb]);
        }
        rs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pop, rs, 0, 0, 0);
      }
    }
    l += rs[0];
    wait_dma();
    __syncthreads();
  };

  int t = 0;
  for (; t + 1 < nb; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    step(t + 1, std::integral_constant<int, 1>{});
  }
  if (t < nb) step(t, std::integral_constant<int, 0>{});

  if (qrow < N) {
    const float invl = 1.0f / l;
    float* op = a.out + ((long long)bh * N + qrow) * kD;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int c0 = 32 * cb + 8 * a4 + 4 * g;
        float4 val;
        val.x = o[cb][4 * a4 + 0] * invl;
        val.y = o[cb][4 * a4 + 1] * invl;
        val.z = o[cb][4 * a4 + 2] * invl;
        val.w = o[cb][4 * a4 + 3] * invl;
        *reinterpret_cast<float4*>(op + c0) = val;
      }
  }
}

}  // namespace vc

using namespace vc;

extern "C" size_t vc_attn_bf16_workspace(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d != kD) return 0;
  const long long nb = (N + kBlock - 1) / kBlock;
  return (size_t)B * H * nb * kTileB;
}

extern "C" int vc_attn_bf16_fwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int B, int H, int N,
                                int d, float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (d != kD) return VC_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !out || B < 1 || H < 1 || N < 1) return VC_ERR_INVALID_ARG;
  if ((long long)B * H > 65535) return VC_ERR_INVALID_ARG;
  const int nb = (N + kBlock - 1) / kBlock;
  const int nqb = (N + 255) / 256;
  if ((long long)nqb * B * H > 0x7FFFFFFFLL) return VC_ERR_INVALID_ARG;
  if ((long long)nb * kTileB > 0xFFFFFFFFLL) return VC_ERR_INVALID_ARG;   // a head's K rows / V^T tiles in one buffer record
  const size_t need = vc_attn_bf16_workspace(B, H, N, d);
  if (!workspace || workspace_bytes < need) return VC_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint16_t* vt = static_cast<uint16_t*>(workspace);
  hipLaunchKernelGGL(transpose_v_bf16, dim3(nb, B * H), dim3(256), 0, st, V, N, nb, vt);
  B16Args a{Q, K, vt, out, N, nb, nqb, B * H, score_scale_c0(softmax_scale)};
  hipLaunchKernelGGL(attn_bf16_kernel, dim3((unsigned)(nqb * B * H)), dim3(kB16Threads), 0, st, a);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? VC_OK : vc_set_hip_error((int)e);
}
