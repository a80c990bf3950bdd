// Fused gather + block mean + quantisation on gfx950.
//
// Method: paper digest "VC-Attention: Value Smoothing and Softmax Casting for
// Low-bit Attention", V-Smooth paragraph (each 128-row hardware block subtracts
// its mean, only the residual is quantised: per-channel E4M3 on the 8-bit path,
// NVFP4 on the 4-bit path; the mean is a 16-bit vector) and preprocessing
// paragraph (mean, gather and quantisation run fused and no high-precision
// intermediate goes back to memory).  News article "Nunchux open-sources
// VC-Attention", section "V-Smooth", item Demean.
//
// The per-channel V scale needs the amax of the residual over all N tokens of a
// (batch, head), so the work is two HBM-streaming passes:
//   pass 1 (one workgroup per permuted 128-row block): gather V rows, block mean
//          (fp32 sum in row order, divided by the row count, bf16 RNE), residual
//          amax per channel -> atomic max (E4M3) or per head (NVFP4)
//   pass 2 (one workgroup per block): gather K and V again, K per-block E4M3,
//          V residual codes (E4M3 with the per-channel scale, or NVFP4), Q
//          per-block E4M3 in original order.  Q and K rows stay in registers,
//          optionally through RoPE and the Hadamard transform first (the same
//          paragraph lists both among the fused steps).  V codes are written transposed
//          per block (channel-major), the operand order of the attention kernel.
// A small clear kernel zeroes the amax accumulators first (no memset on the
// stream, so the sequence can be captured in a graph).
#include <mutex>

#include "vc_common.h"

namespace vc {

constexpr int kRowChunks = kD * 2 / 16;   // 16-byte chunks per bf16 row (16)

// Stage rows of a bf16 [*, 128] tensor into LDS (row r <- src row idx[r]); rows
// >= n are zero.  Every thread moves 16-byte chunks.
// Staged rows keep their 16-byte chunk m at chunk m ^ ((r >> 4) & 7): the
// transposing reads of a wavefront (eight rows 16 apart, one chunk) then fall on
// eight different chunks and no two lanes share an LDS bank.
__device__ __forceinline__ int tile_at(int r, int c) {
  return r * kD + ((((c >> 3) ^ ((r >> 4) & 7)) << 3) | (c & 7));
}

__device__ __forceinline__ void stage_rows(uint16_t* lds, const uint16_t* __restrict__ src,
                                           const int32_t* rows, int n, int nthreads) {
  for (int q = threadIdx.x; q < kBlock * kRowChunks; q += nthreads) {
    const int r = q / kRowChunks, ch = q % kRowChunks;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < n) v = *reinterpret_cast<const uint4*>(src + (long long)rows[r] * kD + ch * 8);
    *reinterpret_cast<uint4*>(lds + tile_at(r, ch * 8)) = v;
  }
}

__global__ void clear_f32(float* p, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// Pass 1: block means and residual amax.  One wavefront per 128-row block, lane
// l on channels 2l and 2l + 1: every permuted row is one 256-byte load and all
// 128 are in flight at once.  Each channel's sum runs over the rows in ascending
// position, in fp32 from 0.  The residual amax max_r |v_r - mu| comes from the
// channel's max and min: rounding is monotone and fl(a - b) = -fl(b - a), so
// max(fl(vmax - mu), fl(mu - vmin), 0) is the same number.
template <int kVFmt>
__global__ void __launch_bounds__(64) pre_pass1(const uint16_t* __restrict__ V, const int32_t* __restrict__ perm,
                                               int N, int nb, uint16_t* __restrict__ means,
                                               float* __restrict__ amax) {
  const int t = blockIdx.x, bh = blockIdx.y, l = threadIdx.x;
  const int n = min(kBlock, N - t * kBlock);
  const int32_t* __restrict__ pr = perm + (long long)bh * N + (long long)t * kBlock;
  const int p0 = pr[l < n ? l : 0], p1 = pr[l + 64 < n ? l + 64 : 0];
  // the head's rows through a buffer resource: the row offset is a scalar, so a
  // load costs one register (its result)
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(V + (long long)bh * N * kD), (short)0, (int)((uint32_t)N * kD * 2u), 0x00020000);
  uint32_t x[kBlock];
#pragma unroll
  for (int r = 0; r < kBlock; ++r) {
    const int row = __builtin_amdgcn_readlane(r < 64 ? p0 : p1, r & 63);
    x[r] = __builtin_amdgcn_raw_buffer_load_b32(vr, 4 * l, (int)((uint32_t)row * (kD * 2u)), 0);
  }
  float s0 = 0.0f, s1 = 0.0f;
  float hi0 = __uint_as_float(x[0] << 16), lo0 = hi0;
  float hi1 = __uint_as_float(x[0] & 0xFFFF0000u), lo1 = hi1;
  // rows past n hold row 0 again: harmless for max and min, and they add +0 to
  // the sums (which start at +0 and so are never -0: s + 0 is s)
#pragma unroll
  for (int r = 0; r < kBlock; ++r) {
    const float v0 = __uint_as_float(x[r] << 16), v1 = __uint_as_float(x[r] & 0xFFFF0000u);
    s0 += r < n ? v0 : 0.0f;
    s1 += r < n ? v1 : 0.0f;
    hi0 = fmaxf(hi0, v0); lo0 = fminf(lo0, v0);
    hi1 = fmaxf(hi1, v1); lo1 = fminf(lo1, v1);
  }
  const uint32_t m0 = f32_to_bf16_rne(s0 / (float)n), m1 = f32_to_bf16_rne(s1 / (float)n);
  reinterpret_cast<uint32_t*>(means + ((long long)bh * nb + t) * kD)[l] = m0 | (m1 << 16);
  const float mu0 = bf16_bits_to_f32(m0), mu1 = bf16_bits_to_f32(m1);
  // + 0 and the sign clear keep a -0 out of the unsigned-ordered atomic max
  const float a0 = __uint_as_float(__float_as_uint(fmaxf(fmaxf(hi0 - mu0, mu0 - lo0), 0.0f)) & 0x7FFFFFFFu);
  const float a1 = __uint_as_float(__float_as_uint(fmaxf(fmaxf(hi1 - mu1, mu1 - lo1), 0.0f)) & 0x7FFFFFFFu);
  if (kVFmt == VC_V_E4M3) {
    atomic_max_nonneg(&amax[(long long)bh * kD + 2 * l], a0);
    atomic_max_nonneg(&amax[(long long)bh * kD + 2 * l + 1], a1);
  } else {
    float am = fmaxf(a0, a1);
    for (int o = 32; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o));
    if (l == 0) atomic_max_nonneg(&amax[bh], am);
  }
}

// Half of a bf16 row (channels 64p .. 64p + 63) as 32 packed words (zero when
// the row is past the block's end).
__device__ __forceinline__ void load_half_row(const uint16_t* __restrict__ src, int row, bool valid, int p,
                                              uint32_t (&w)[32]) {
  if (valid) {
    const uint4* rp = reinterpret_cast<const uint4*>(src + (long long)row * kD + 64 * p);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 u = rp[j];
      w[4 * j] = u.x; w[4 * j + 1] = u.y; w[4 * j + 2] = u.z; w[4 * j + 3] = u.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i] = 0u;
  }
}

// Q or K rows (optionally) through RoPE and the Walsh-Hadamard transform, then
// per-block E4M3 with scale = amax/448, all in registers: thread 2r + p holds channels 64p .. 64p + 63 of row r
// (256 threads, 128 rows; the words come from load_half_row).  Arithmetic in fp32, in the order of the method's
// reading: RoPE on channel pairs (2i, 2i+1) with the caller's (cos, sin) of the
// row's original position, y0 = fmaf(x0, c, -(x1 s)), y1 = fmaf(x0, s, x1 c);
// the unnormalised Sylvester transform stage by stage (h = 1 .. 32 inside a
// thread, h = 64 across the thread pair), (a + b, a - b); K rows then scaled by
// 2^-7 so that Q' . K' = Q . K.  Block scale amax/448, codes E4M3(y * 448/amax).
__device__ __forceinline__ void transform_encode(const uint32_t (&w32)[32], int src_row, int n,
                                 const float2* __restrict__ rope, bool hadamard, bool k_side,
                                 uint8_t* __restrict__ out_rows, float* __restrict__ scale_out, float* red) {
  const int tid = threadIdx.x, r = tid >> 1, p = tid & 1;
  const bool valid = r < n;
  float y[64];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    y[2 * e] = __uint_as_float(w32[e] << 16);
    y[2 * e + 1] = __uint_as_float(w32[e] & 0xFFFF0000u);
  }
  if (rope && valid) {
    const float2* cs = rope + (long long)src_row * 64 + 32 * p;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float2 c = cs[i];
      const float x0 = y[2 * i], x1 = y[2 * i + 1];
      y[2 * i] = __builtin_fmaf(x0, c.x, -(x1 * c.y));
      y[2 * i + 1] = __builtin_fmaf(x0, c.y, x1 * c.x);
    }
  }
  if (hadamard) {
#pragma unroll
    for (int h = 1; h < 64; h *= 2)
#pragma unroll
      for (int i = 0; i < 64; ++i)
        if ((i & h) == 0) {
          const float a = y[i], b = y[i + h];
          y[i] = a + b;
          y[i + h] = a - b;
        }
#pragma unroll
    for (int i = 0; i < 64; ++i) {   // h = 64: channel i (thread p = 0) with channel i + 64 (p = 1)
      const float o = __shfl_xor(y[i], 1);
      y[i] = p == 0 ? y[i] + o : o - y[i];
      if (k_side) y[i] *= 0x1p-7f;
    }
  }
  float am = 0.0f;
  if (valid)
#pragma unroll
    for (int i = 0; i < 64; ++i) am = fmaxf(am, fabsf(y[i]));
  for (int o = 32; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o));
  if ((tid & 63) == 0) red[tid >> 6] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = am > 0.0f ? 448.0f / am : 0.0f;
  if (tid == 0) *scale_out = am > 0.0f ? am / 448.0f : 0.0f;
  uint32_t w[16];
#pragma unroll
  for (int e = 0; e < 16; ++e)
    w[e] = valid ? pack2_e4m3_sat<true>(y[4 * e + 2] * inv, y[4 * e + 3] * inv,
                                        pack2_e4m3_sat<false>(y[4 * e] * inv, y[4 * e + 1] * inv, 0u))
                 : 0u;
  uint8_t* op = out_rows + (long long)r * kD + 64 * p;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<uint4*>(op + 16 * j) = make_uint4(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]);
  __syncthreads();
}

__device__ __forceinline__ uint32_t e2m1_rne_sat(float x) {
  const float a = fminf(fabsf(x), 6.0f);
  float q;
  if (a < 2.0f) q = __builtin_rintf(a * 2.0f) * 0.5f;
  else if (a < 4.0f) q = __builtin_rintf(a);
  else q = __builtin_rintf(a * 0.5f) * 2.0f;
  q = fminf(q, 6.0f);
  uint32_t idx = q < 2.0f ? (uint32_t)(q * 2.0f) : (q < 4.0f ? 2u + (uint32_t)q : (q < 6.0f ? 6u : 7u));
  return idx | ((__float_as_uint(x) >> 28) & 8u);
}

template <int kVFmt>
__global__ void __launch_bounds__(256) pre_pass2(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                 const uint16_t* __restrict__ V, const int32_t* __restrict__ perm,
                                                 int N, int nb, const float* __restrict__ amax,
                                                 const uint16_t* __restrict__ means,
                                                 uint8_t* __restrict__ q_codes, float* __restrict__ q_scales,
                                                 uint8_t* __restrict__ k_codes, float* __restrict__ k_scales,
                                                 uint8_t* __restrict__ v_codes, float* __restrict__ v_scales,
                                                 uint8_t* __restrict__ v_gscales, const float2* __restrict__ rope,
                                                 int hadamard) {
  __shared__ __align__(16) uint16_t tile[kBlock * kD];
  __shared__ int32_t rows[kBlock];
  __shared__ float red[4];
  __shared__ float aux[kD];   // E4M3: 448/amax_c ; NVFP4 unused
  const int t = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int n = min(kBlock, N - t * kBlock);
  const long long rowbase = (long long)bh * nb * kBlock + (long long)t * kBlock;  // padded row index
  if (tid < kBlock) rows[tid] = tid < n ? perm[(long long)bh * N + t * kBlock + tid] : 0;
  __syncthreads();

  // Every load of the block is issued before any is used, so that the K rows,
  // the V rows and the Q rows (96 KiB) are in flight together: K and Q half rows
  // into registers, V rows straight into the swizzled LDS tile (global -> LDS
  // copies; rows past n read as zero through the buffer's record count).
  const int r = tid >> 1, p = tid & 1;
  uint32_t kw[32], qw[32];
  load_half_row(K + (long long)bh * N * kD, rows[r], r < n, p, kw);
  {
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(V + (long long)bh * N * kD), (short)0, (int)((uint32_t)N * kD * 2u), 0x00020000);
    const int wave = tid >> 6, lane = tid & 63;
    uint32_t off[8], src[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) src[j] = (uint32_t)rows[(wave * 8 + j) * 4 + (lane >> 4)];
    // rows[] is 0 past n: read unconditionally (no branch around the reads)
    asm volatile("" : "+v"(src[0]), "+v"(src[1]), "+v"(src[2]), "+v"(src[3]), "+v"(src[4]), "+v"(src[5]),
                 "+v"(src[6]), "+v"(src[7]));
#pragma unroll
    for (int j = 0; j < 8; ++j) {   // 16-byte LDS chunk (wave * 8 + j) * 64 + lane of the tile
      const int rr = (wave * 8 + j) * 4 + (lane >> 4), m = (lane & 15) ^ ((rr >> 4) & 7);
      off[j] = rr < n ? src[j] * (kD * 2u) + 16u * m : 0xFFFFFFF0u;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          vr, (__attribute__((address_space(3))) void*)(reinterpret_cast<uint8_t*>(tile) + (wave * 8 + j) * 1024),
          16, (int)off[j], 0, 0, 0);
  }
  if (Q) load_half_row(Q + (long long)bh * N * kD, t * kBlock + r, r < n, p, qw);

  // K: gathered, per-block scale
  transform_encode(kw, rows[r], n, rope, hadamard != 0, true, k_codes + rowbase * kD,
                   k_scales + (long long)bh * nb + t, red);

  // V residual
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (kVFmt == VC_V_E4M3) {
    if (tid < kD) {
      const float am = amax[(long long)bh * kD + tid];
      aux[tid] = am > 0.0f ? 448.0f / am : 0.0f;
      if (t == 0) v_scales[(long long)bh * kD + tid] = am > 0.0f ? am / 448.0f : 0.0f;
    }
    __syncthreads();
    // channel c, rows u0..u0+15 -> 16 bytes of the transposed block
    for (int q = tid; q < kD * 8; q += 256) {
      const int c = q >> 3, u0 = (q & 7) * 16;
      const float mu = bf16_bits_to_f32(means[((long long)bh * nb + t) * kD + c]);
      const float inv = aux[c];
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x[4];
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          const int u = u0 + 4 * e + z;
          x[z] = u < n ? (bf16_bits_to_f32(tile[tile_at(u, c)]) - mu) * inv : 0.0f;
        }
        w[e] = pack2_e4m3_sat<true>(x[2], x[3], pack2_e4m3_sat<false>(x[0], x[1], 0u));
        if (u0 + 4 * e >= n) w[e] = 0u;   // padding rows are zero bytes (not -0)
        else {
#pragma unroll
          for (int z = 1; z < 4; ++z)
            if (u0 + 4 * e + z >= n) w[e] &= ~(0xFFu << (8 * z));
        }
      }
      *reinterpret_cast<uint4*>(v_codes + (((long long)bh * nb + t) * kD + c) * kBlock + u0) =
          make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else if (kVFmt == VC_V_MXFP4) {
    // MXFP4: E2M1 values, one E8M0 scale per group of 32 rows of a channel:
    // group (h, g) = rows 64h + 16g + [0, 16) and 64h + 32 + 16g + [0, 16),
    // the values one lane of the block-scaled FP4 MFMA holds.  Scale code
    // floor(log2 amax) - 2 + 127 (the exponent field of amax minus 2, clamped
    // at 0); values E2M1_RNE_SAT(R * 2^(127 - code)), an exact scaling.
    if (t == 0 && tid < kD) v_scales[(long long)bh * kD + tid] = 1.0f;
    for (int q = tid; q < kD * 4; q += 256) {
      const int c = q >> 2, h = (q >> 1) & 1, gg = q & 1;
      const float mu = bf16_bits_to_f32(means[((long long)bh * nb + t) * kD + c]);
      float r[32];
      float gam = 0.0f;
#pragma unroll
      for (int z = 0; z < 32; ++z) {
        const int u = 64 * h + 16 * gg + (z < 16 ? z : 16 + z);
        r[z] = u < n ? bf16_bits_to_f32(tile[tile_at(u, c)]) - mu : 0.0f;
        gam = fmaxf(gam, fabsf(r[z]));
      }
      const int eb = (int)((__float_as_uint(gam) >> 23) & 0xFFu);
      const int code = eb >= 2 ? eb - 2 : 0;
      const float xinv = __uint_as_float((uint32_t)(254 - code) << 23);
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int z = 0; z < 32; ++z) w[z >> 3] |= e2m1_rne_sat(r[z] * xinv) << (4 * (z & 7));
      const long long cb = ((long long)bh * nb + t) * kD + c;
      *reinterpret_cast<uint4*>(v_codes + cb * 64 + 32 * h + 16 * gg) = make_uint4(w[0], w[1], w[2], w[3]);
      v_gscales[(cb * 2 + gg) * 2 + h] = (uint8_t)code;
    }
  } else {
    const float St = amax[bh] / 2688.0f;             // amax_all / (6 * 448)
    const float six_st = 6.0f * St;
    if (t == 0 && tid == 0) v_scales[bh] = St;
    // channel c, group of 16 rows u0..u0+15: one E4M3 group scale, 8 packed bytes
    for (int q = tid; q < kD * 8; q += 256) {
      const int c = q >> 3, g = q & 7, u0 = g * 16;
      const float mu = bf16_bits_to_f32(means[((long long)bh * nb + t) * kD + c]);
      float r[16];
      float gam = 0.0f;
#pragma unroll
      for (int z = 0; z < 16; ++z) {
        const int u = u0 + z;
        r[z] = u < n ? bf16_bits_to_f32(tile[tile_at(u, c)]) - mu : 0.0f;
        if (u < n) gam = fmaxf(gam, fabsf(r[z]));
      }
      const uint32_t sg = St > 0.0f ? f32_to_e4m3_sat(gam / six_st) : 0u;
      const float dsg = e4m3_to_f32(sg) * St;
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int z = 0; z < 16; ++z) {
        const uint32_t nib = (u0 + z < n && dsg > 0.0f) ? e2m1_rne_sat(r[z] / dsg) : 0u;
        w[z >> 3] |= nib << (4 * (z & 7));
      }
      *reinterpret_cast<uint2*>(v_codes + (((long long)bh * nb + t) * kD + c) * (kBlock / 2) + u0 / 2) =
          make_uint2(w[0], w[1]);
      v_gscales[((long long)bh * nb * 8 + t * 8 + g) * kD + c] = (uint8_t)sg;
    }
  }
  __syncthreads();

  // Q: original order, per-block scale
  if (Q)
    transform_encode(qw, t * kBlock + r, n, rope, hadamard != 0, false, q_codes + rowbase * kD,
                     q_scales + (long long)bh * nb + t, red);
}

}  // namespace vc

using namespace vc;

extern "C" size_t vc_preprocess_workspace(int B, int H, int N, int d, int v_format) {
  if (B < 1 || H < 1 || N < 1 || d != kD) return 0;
  const long long BH = (long long)B * H;
  return v_format == VC_V_NVFP4 ? (size_t)BH * sizeof(float) : (size_t)BH * kD * sizeof(float);
}

extern "C" int vc_preprocess_quant_ex(const uint16_t* Q, const uint16_t* K, const uint16_t* V, const int32_t* perm,
                                      int B, int H, int N, int d, int v_format, const float* rope_cs, int hadamard,
                                      uint8_t* q_codes, float* q_scales, uint8_t* k_codes, float* k_scales,
                                      uint8_t* v_codes, float* v_scales, uint8_t* v_group_scales, uint16_t* v_means,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (d != kD) return VC_ERR_UNSUPPORTED;
  if (v_format != VC_V_E4M3 && v_format != VC_V_NVFP4 && v_format != VC_V_MXFP4) return VC_ERR_UNSUPPORTED;
  if (!K || !V || !perm || !k_codes || !k_scales || !v_codes || !v_scales || !v_means) return VC_ERR_INVALID_ARG;
  if (Q && (!q_codes || !q_scales)) return VC_ERR_INVALID_ARG;
  if ((v_format == VC_V_NVFP4 || v_format == VC_V_MXFP4) && !v_group_scales) return VC_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || (long long)B * H > 65535) return VC_ERR_INVALID_ARG;
  if ((long long)N * kD * 2 > 0xFFFFFFFFLL) return VC_ERR_INVALID_ARG;   // a head's V rows in one buffer record
  if (hadamard != 0 && hadamard != 1) return VC_ERR_INVALID_ARG;
  const size_t need = vc_preprocess_workspace(B, H, N, d, v_format);
  if (!workspace || workspace_bytes < need) return VC_ERR_WORKSPACE;
  const long long BH = (long long)B * H;
  const int nb = (N + kBlock - 1) / kBlock;
  float* amax = static_cast<float*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const long long na = (long long)(need / sizeof(float));
  const float2* rope = reinterpret_cast<const float2*>(rope_cs);
  hipLaunchKernelGGL(clear_f32, dim3((unsigned)((na + 255) / 256)), dim3(256), 0, st, amax, na);
  const dim3 grid(nb, (unsigned)BH);
  if (v_format == VC_V_E4M3) {
    hipLaunchKernelGGL(pre_pass1<VC_V_E4M3>, grid, dim3(64), 0, st, V, perm, N, nb, v_means, amax);
    hipLaunchKernelGGL(pre_pass2<VC_V_E4M3>, grid, dim3(256), 0, st, Q, K, V, perm, N, nb, amax, v_means,
                       q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, v_group_scales, rope, hadamard);
  } else if (v_format == VC_V_MXFP4) {
    hipLaunchKernelGGL(pre_pass1<VC_V_E4M3>, grid, dim3(64), 0, st, V, perm, N, nb, v_means, amax);
    hipLaunchKernelGGL(pre_pass2<VC_V_MXFP4>, grid, dim3(256), 0, st, Q, K, V, perm, N, nb, amax, v_means,
                       q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, v_group_scales, rope, hadamard);
  } else {
    hipLaunchKernelGGL(pre_pass1<VC_V_NVFP4>, grid, dim3(64), 0, st, V, perm, N, nb, v_means, amax);
    hipLaunchKernelGGL(pre_pass2<VC_V_NVFP4>, grid, dim3(256), 0, st, Q, K, V, perm, N, nb, amax, v_means,
                       q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, v_group_scales, rope, hadamard);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return vc_set_hip_error((int)e);
  return VC_OK;
}

// Scratch of the allocation-free entry point: the amax accumulators live in a
// file-scope device array (one copy per GPU, held until the process ends)
// instead of a caller workspace.  On the host `scratch` only names the symbol;
// its device address comes from hipGetSymbolAddress, looked up once per device.
constexpr size_t kScratchBytes = 1u << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (nullptr and a recorded
// HIP error if the lookup fails).
void* scratch_on_current_device() {
  int dev = 0;
  const hipError_t ed = hipGetDevice(&dev);
  if (ed != hipSuccess) { vc_set_hip_error((int)ed); return nullptr; }
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) { vc_set_hip_error((int)e); return nullptr; }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" size_t vc_preprocess_noalloc_max_scratch(void) { return kScratchBytes; }

extern "C" int vc_preprocess_quant_noalloc(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                           const int32_t* perm, int B, int H, int N, int d, int v_format,
                                           uint8_t* q_codes, float* q_scales, uint8_t* k_codes, float* k_scales,
                                           uint8_t* v_codes, float* v_scales, uint8_t* v_group_scales,
                                           uint16_t* v_means, void* stream) {
  if (d != kD) return VC_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || N < 1) return VC_ERR_INVALID_ARG;
  const size_t need = vc_preprocess_workspace(B, H, N, d, v_format);
  if (need > kScratchBytes) return VC_ERR_SCRATCH;
  if (v_format != VC_V_E4M3 && v_format != VC_V_NVFP4 && v_format != VC_V_MXFP4) return VC_ERR_UNSUPPORTED;
  if (!K || !V || !perm || !k_codes || !k_scales || !v_codes || !v_scales || !v_means) return VC_ERR_INVALID_ARG;
  void* ws = scratch_on_current_device();
  if (!ws) return VC_ERR_HIP;
  // the clear kernel inside zeroes the accumulators first on every call
  return vc_preprocess_quant_ex(Q, K, V, perm, B, H, N, d, v_format, nullptr, 0, q_codes, q_scales, k_codes,
                                k_scales, v_codes, v_scales, v_group_scales, v_means, ws, kScratchBytes, stream);
}

extern "C" int vc_preprocess_quant(const uint16_t* Q, const uint16_t* K, const uint16_t* V, const int32_t* perm,
                                   int B, int H, int N, int d, int v_format, uint8_t* q_codes, float* q_scales,
                                   uint8_t* k_codes, float* k_scales, uint8_t* v_codes, float* v_scales,
                                   uint8_t* v_group_scales, uint16_t* v_means, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return vc_preprocess_quant_ex(Q, K, V, perm, B, H, N, d, v_format, nullptr, 0, q_codes, q_scales, k_codes,
                                k_scales, v_codes, v_scales, v_group_scales, v_means, workspace, workspace_bytes,
                                stream);
}
