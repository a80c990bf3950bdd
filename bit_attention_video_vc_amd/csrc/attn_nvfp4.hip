// 4-bit V-Smooth attention on gfx950: NVFP4 V residual, fp32 softmax, bf16 P.
//
// Method: paper digest "VC-Attention: Value Smoothing and Softmax Casting for
// Low-bit Attention", V-Smooth paragraph (the 4-bit path quantises the block
// residual to NVFP4) and preprocessing paragraph (ExpCast is not used on the
// 4-bit path: NVFP4 has no single affine log-to-code map, softmax stays fp32).
//
// MI355X has no NVFP4 matrix instruction, so P.V runs as a bf16 MFMA on the
// exactly dequantised residual: E2M1 value x E4M3 group scale has at most six
// significant bits and is exact in bf16; the per-(batch, head) fp32 scale St is
// applied in the epilogue.  Q.K stays FP8 (the same transposed-score scheme as
// the 8-bit kernel), P = exp2(S*kap - mx) in fp32 rounded to bf16, row sums of
// the rounded P, block means restored with the batched rank-2 fp32 MFMA.
#include <type_traits>

#include "attn_common.h"

namespace vc {

constexpr int kN4Threads = 256;
constexpr int kRowBf = kD * 2;   // bytes per bf16 V^T row (256)
constexpr int kTile_ = kBlock * kD;   // bytes of one FP8 K tile

struct N4Args {
  const uint8_t* q;  const float* qs;
  const uint8_t* k;  const float* ks;
  const uint8_t* v;  const float* vs;   // nibbles [BH, nb, 128, 64]; St [BH]
  const uint8_t* gs;                    // E4M3 group scales [BH, Np/16, 128]
  const uint16_t* means;
  float* out;
  float* sdump; uint16_t* pdump;        // test hook: scores and bf16 P bits [BH, N, Np] (or null)
  int N, nb, BH;
  float c0;
};

__device__ __forceinline__ v16f mfma_bf16x(const v8bf& a, const v8bf& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// E2M1 nibble -> fp32 (sign, 2 exponent bits with bias 1, 1 mantissa bit).
__device__ __forceinline__ float e2m1_to_f32(uint32_t n) {
  const uint32_t e = (n >> 1) & 3u, m = n & 1u;
  const uint32_t mag = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3F000000u : 0u);
  return __uint_as_float(mag | ((n & 8u) << 28));
}

template <bool kDump>
__global__ void __launch_bounds__(kN4Threads) attn_nvfp4_kernel(N4Args a) {
  __shared__ __align__(16) uint8_t Ks[kTile_];
  __shared__ __align__(16) uint8_t Vb[kD * kRowBf];    // dequantised V^T, bf16, swizzled
  __shared__ __align__(16) float MuT[kD];
  __shared__ float InvSt;

  const int nqb = a.nb;
  const int item = xcd_item(blockIdx.x, nqb * a.BH);
  const int bh = item / nqb, qb = item % nqb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, col = lane & 31;
  const int N = a.N, nb = a.nb;
  const long long Np = (long long)nb * kBlock;
  const float St = a.vs[bh];
  const float Stp = St > 0.0f ? St : 1.0f;
  if (tid == 0) InvSt = 1.0f / Stp;

  const int qrow = qb * kBlock + wave * 32 + col;
  v8i qop[2];
  {
    const uint8_t* qp = a.q + ((long long)bh * Np + qrow) * kD;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const uint4 lo = *reinterpret_cast<const uint4*>(qp + 64 * c2 + 32 * g);
      const uint4 hi = *reinterpret_cast<const uint4*>(qp + 64 * c2 + 32 * g + 16);
      qop[c2][0] = lo.x; qop[c2][1] = lo.y; qop[c2][2] = lo.z; qop[c2][3] = lo.w;
      qop[c2][4] = hi.x; qop[c2][5] = hi.y; qop[c2][6] = hi.z; qop[c2][7] = hi.w;
    }
  }
  const float sq = a.qs[(long long)bh * nb + qb];
  const uint8_t* kbase = a.k + (long long)bh * Np * kD;
  const uint8_t* vbase = a.v + (long long)bh * nb * kD * 64;
  const uint8_t* gbase = a.gs + (long long)bh * nb * 8 * kD;
  const uint16_t* mbase = a.means + (long long)bh * nb * kD;

  v16f o[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[cb][r] = 0.0f;
  float mx = -__builtin_inff(), l = 0.0f;
  float abat = 0.0f, mbat[4] = {0.0f, 0.0f, 0.0f, 0.0f};

  for (int t = 0; t < nb; ++t) {
    __syncthreads();   // previous tile's LDS reads are done
    // K tile straight to LDS (same swizzle as the 8-bit kernel)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 4 * i + wave;
      const int row = 8 * j + (lane >> 3), pos = lane & 7;
      dma16(kbase + (long long)t * kTile_ + row * kD + 16 * (pos ^ swz_k(row)), &Ks[1024 * j]);
    }
    // V: thread -> (channel tid/2, rows 64*(tid&1) .. +63), dequantised to bf16
    {
      const int ch = tid >> 1, half = tid & 1;
      const uint8_t* np_ = vbase + ((long long)t * kD + ch) * 64 + 32 * half;
      const uint4 n0 = *reinterpret_cast<const uint4*>(np_);
      const uint4 n1 = *reinterpret_cast<const uint4*>(np_ + 16);
      const uint32_t nw[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {          // 4 groups of 16 rows
        const float sc = e4m3_to_f32(gbase[((long long)t * 8 + 4 * half + gi) * kD + ch]);
        uint32_t packed[8];
#pragma unroll
        for (int z = 0; z < 16; z += 2) {
          const uint32_t w = nw[2 * gi + (z >> 3)];
          const uint32_t b0 = (w >> (4 * (z & 7))) & 15u, b1 = (w >> (4 * ((z + 1) & 7))) & 15u;
          const uint32_t v0 = __float_as_uint(e2m1_to_f32(b0) * sc) >> 16;   // exact in bf16
          const uint32_t v1 = __float_as_uint(e2m1_to_f32(b1) * sc) >> 16;
          packed[z >> 1] = v0 | (v1 << 16);
        }
        const int key0 = 64 * half + 16 * gi;     // 16 keys = two 16-byte chunks
#pragma unroll
        for (int hc = 0; hc < 2; ++hc) {
          const int chunk = (key0 >> 3) + hc;
          *reinterpret_cast<uint4*>(&Vb[ch * kRowBf + 16 * (chunk ^ (ch & 15))]) =
              make_uint4(packed[4 * hc], packed[4 * hc + 1], packed[4 * hc + 2], packed[4 * hc + 3]);
        }
      }
    }
    if (tid < kD) MuT[(tid & 31) * 4 + (tid >> 5)] = bf16_bits_to_f32(mbase[(long long)t * kD + tid]) * InvSt;
    wait_dma();
    __syncthreads();

    v16f s[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[m][r] = 0.0f;
      const int row = sigma(m, col);
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) s[m] = mfma32(lds_op(&Ks[row * kD], 4 * c2 + 2 * g, swz_k(row)), qop[c2], s[m]);
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
    const float kap = (sq * a.ks[(long long)bh * nb + t]) * a.c0;
    const float mx_new = fmaxf(mx, M * kap);
    const float alpha = __builtin_amdgcn_exp2f(mx - mx_new);
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[cb][r] *= alpha;
    }
    l *= alpha;
    abat *= alpha;
    mx = mx_new;

    // keys at or beyond N (last tile only) get P = 0: their scores are -inf
    // for the row max, and -inf * kap is NaN when kap = 0 (a zero Q or K block)
    const int nvalid = min(N - t * kBlock, kBlock);
    float rsum = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        uint32_t pw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key0 = 64 * (m >> 1) + 32 * g + 16 * (m & 1) + 8 * s2 + 2 * e;
          float p0 = __builtin_amdgcn_exp2f(s[m][8 * s2 + 2 * e] * kap - mx_new);
          float p1 = __builtin_amdgcn_exp2f(s[m][8 * s2 + 2 * e + 1] * kap - mx_new);
          if (nvalid < kBlock) {
            p0 = key0 < nvalid ? p0 : 0.0f;
            p1 = key0 + 1 < nvalid ? p1 : 0.0f;
          }
          const uint32_t b0 = f32_to_bf16_rne(p0), b1 = f32_to_bf16_rne(p1);
          if (kDump && qrow < N) {
            const long long idx = ((long long)bh * N + qrow) * Np + (long long)t * kBlock + key0;
            a.sdump[idx] = key0 < nvalid ? s[m][8 * s2 + 2 * e] : 0.0f;
            a.sdump[idx + 1] = key0 + 1 < nvalid ? s[m][8 * s2 + 2 * e + 1] : 0.0f;
            a.pdump[idx] = (uint16_t)b0;
            a.pdump[idx + 1] = (uint16_t)b1;
          }
          rsum += __uint_as_float(b0 << 16) + __uint_as_float(b1 << 16);
          pw[e] = b0 | (b1 << 16);
        }
        v8bf pop;
        __builtin_memcpy(&pop, pw, 16);
        const int keyoff = 64 * (m >> 1) + 32 * g + 16 * (m & 1) + 8 * s2;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int ch = 32 * cb + col;
          v8bf vv;
          __builtin_memcpy(&vv, &Vb[ch * kRowBf + 16 * ((keyoff >> 3) ^ (ch & 15))], 16);
          o[cb] = mfma_bf16x(vv, pop, o[cb]);
        }
      }
    rsum += __shfl_xor(rsum, 32);
    l += rsum;
    {
      const float4 mu = *reinterpret_cast<const float4*>(&MuT[col * 4]);
      const bool mine = g == (t & 1);
      abat = mine ? rsum : abat;
      mbat[0] = mine ? mu.x : mbat[0];
      mbat[1] = mine ? mu.y : mbat[1];
      mbat[2] = mine ? mu.z : mbat[2];
      mbat[3] = mine ? mu.w : mbat[3];
      if ((t & 1) || t + 1 == nb) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          o[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(mbat[cb], abat, o[cb], 0, 0, 0);
        abat = 0.0f;
      }
    }
  }

  if (qrow < N) {
    const float sc = Stp / l;
    float* op = a.out + ((long long)bh * N + qrow) * kD;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int c0 = 32 * cb + 8 * a4 + 4 * g;
        float4 val;
        val.x = o[cb][4 * a4 + 0] * sc;
        val.y = o[cb][4 * a4 + 1] * sc;
        val.z = o[cb][4 * a4 + 2] * sc;
        val.w = o[cb][4 * a4 + 3] * sc;
        *reinterpret_cast<float4*>(op + c0) = val;
      }
  }
}

}  // namespace vc

using namespace vc;

int vc_attn_nvfp4_launch(const uint8_t* q_codes, const float* q_scales, const uint8_t* k_codes,
                         const float* k_scales, const uint8_t* v_codes, const float* v_scales,
                         const uint8_t* v_group_scales, const uint16_t* v_means, int B, int H, int N,
                         float c0, float* out, float* s_dump, uint16_t* p_dump, hipStream_t st) {
  const int nb = (N + kBlock - 1) / kBlock;
  N4Args a{q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, v_group_scales, v_means, out,
           s_dump, p_dump, N, nb, B * H, c0};
  const dim3 grid((unsigned)(nb * B * H)), block(kN4Threads);
  if (s_dump) hipLaunchKernelGGL(attn_nvfp4_kernel<true>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(attn_nvfp4_kernel<false>, grid, block, 0, st, a);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? VC_OK : vc_set_hip_error((int)e);
}
