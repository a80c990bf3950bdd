// Comparator: standard non-causal flash attention in bf16 on gfx950.
//
// The pages quote every attention speed-up against BF16 FlashAttention-4
// (insight article, section "A Faster Kernel Does Not Automatically Mean
// Faster Generation"; paper digest, results table).  This kernel is the in-repo
// stand-in on MI355X: bf16 V_MFMA_F32_32X32X16_BF16 for Q.K^T and P.V, online
// softmax with fp32 exp2, P rounded to bf16 (round to nearest even), row sums
// of the rounded P.
//
// Same lane organisation as the FP8 kernel: S^T = K.Q^T so that each lane holds
// one query's scores and the bf16 P values are already in the B-operand layout
// of O^T = V^T.P^T.  V is transposed into LDS while it is staged.
#include "attn_common.h"

namespace vc {

constexpr int kB16Threads = 256;
constexpr int kRowB = kD * 2;   // bytes per bf16 row (256)

typedef short v4s __attribute__((ext_vector_type(4)));

struct B16Args {
  const uint16_t* q; const uint16_t* k; const uint16_t* v;
  float* out;
  int N, nb, BH;
  float c0;
};

__device__ __forceinline__ int swz_kb(int row) {
  return (row & 3) | (((row >> 2) & 1) << 2) | (((row >> 5) & 1) << 3);
}
__device__ __forceinline__ int swz_vb(int row) { return row & 15; }

__device__ __forceinline__ v16f mfma_bf16(const v8bf& a, const v8bf& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf as_bf(uint4 u) {
  v8bf r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

__global__ void __launch_bounds__(kB16Threads) attn_bf16_kernel(B16Args a) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* Kt = smem;                     // [2][128 keys][256 B]
  uint8_t* Vt = smem + 2 * kBlock * kRowB; // [2][128 ch][256 B] (transposed)

  const int nqb = a.nb;
  const int item = xcd_item(blockIdx.x, nqb * a.BH);
  const int bh = item / nqb, qb = item % nqb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, col = lane & 31;
  const int N = a.N, nb = a.nb;

  const int qrow = qb * kBlock + wave * 32 + col;
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
  const uint16_t* kbase = a.k + (long long)bh * N * kD;
  const uint16_t* vbase = a.v + (long long)bh * N * kD;

  // K tile: global -> LDS directly (instruction j of 32 fills LDS bytes
  // [1024j, 1024j+1024): lane i writes row 4j + i/16 at chunk position i%16).
  // V tile: staged through registers and written transposed.
  auto load_k = [&](int t, int buf) {
    uint8_t* K = Kt + buf * kBlock * kRowB;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = 4 * i + wave;
      const int row = 4 * j + (lane >> 4), pos = lane & 15;
      const int key = min(t * kBlock + row, N - 1);   // rows past N are masked later
      dma16(kbase + (long long)key * kD + 8 * (pos ^ swz_kb(row)), K + 1024 * j);
    }
  };
  uint4 vr[8];
  auto load_v = [&](int t) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int qd = tid + kB16Threads * i;
      const int vkey_local = qd & 127, vch = qd >> 7;          // consecutive keys per wave
      const int vkey = t * kBlock + vkey_local;
      vr[i] = vkey < N ? *reinterpret_cast<const uint4*>(vbase + (long long)vkey * kD + 8 * vch)
                       : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_v = [&](int buf) {
    uint8_t* V = Vt + buf * kBlock * kRowB;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int qd = tid + kB16Threads * i;
      const int key = qd & 127, c0 = 8 * (qd >> 7);
      const uint32_t w[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = c0 + e;
        const uint16_t val = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        *reinterpret_cast<uint16_t*>(V + c * kRowB + 16 * ((key >> 3) ^ swz_vb(c)) + 2 * (key & 7)) = val;
      }
    }
  };

  load_k(0, 0);
  load_v(0);
  store_v(0);
  wait_dma();
  __syncthreads();

  v16f o[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[cb][r] = 0.0f;
  float mx = -__builtin_inff(), l = 0.0f;

  for (int t = 0; t < nb; ++t) {
    const int buf = t & 1;
    const uint8_t* K = Kt + buf * kBlock * kRowB;
    const uint8_t* V = Vt + buf * kBlock * kRowB;
    if (t + 1 < nb) load_k(t + 1, buf ^ 1);

    v16f s[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[m][r] = 0.0f;
      const int row = sigma(m, col);
      const uint8_t* rb = K + row * kRowB;
      const int sw = swz_kb(row);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        s[m] = mfma_bf16(as_bf(*reinterpret_cast<const uint4*>(rb + 16 * ((2 * j + g) ^ sw))), qop[j], s[m]);
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

    if (t + 1 < nb) load_v(t + 1);
    float rsum = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        uint32_t pw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(s[m][8 * s2 + 2 * e] * a.c0 - mx_new);
          const float p1 = __builtin_amdgcn_exp2f(s[m][8 * s2 + 2 * e + 1] * a.c0 - mx_new);
          const uint32_t b0 = f32_to_bf16_rne(p0), b1 = f32_to_bf16_rne(p1);
          rsum += __uint_as_float(b0 << 16) + __uint_as_float(b1 << 16);
          pw[e] = b0 | (b1 << 16);
        }
        const v8bf pop = as_bf(make_uint4(pw[0], pw[1], pw[2], pw[3]));
        const int keyoff = 64 * (m >> 1) + 32 * g + 16 * (m & 1) + 8 * s2;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int ch = 32 * cb + col;
          const uint4 vv = *reinterpret_cast<const uint4*>(V + ch * kRowB + 16 * ((keyoff >> 3) ^ swz_vb(ch)));
          o[cb] = mfma_bf16(as_bf(vv), pop, o[cb]);
        }
      }
    }
    rsum += __shfl_xor(rsum, 32);
    l += rsum;

    if (t + 1 < nb) store_v(buf ^ 1);
    wait_dma();
    __syncthreads();
  }

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

extern "C" int vc_attn_bf16_fwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int B, int H, int N,
                                int d, float softmax_scale, float* out, void* stream) {
  if (d != kD) return VC_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !out || B < 1 || H < 1 || N < 1) return VC_ERR_INVALID_ARG;
  const int nb = (N + kBlock - 1) / kBlock;
  if ((long long)nb * B * H > 0x7FFFFFFFLL) return VC_ERR_INVALID_ARG;
  B16Args a{Q, K, V, out, N, nb, B * H, score_scale_c0(softmax_scale)};
  const size_t lds = 4u * kBlock * kRowB;   // 128 KiB: double-buffered K and V^T
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(attn_bf16_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr_set = true;
  }
  hipLaunchKernelGGL(attn_bf16_kernel, dim3((unsigned)(nb * B * H)), dim3(kB16Threads), lds,
                     static_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? VC_OK : vc_set_hip_error((int)e);
}
