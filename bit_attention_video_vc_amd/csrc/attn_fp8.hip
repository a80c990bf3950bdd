// Non-causal FP8 flash attention with V-Smooth mean restore and ExpCast-FP8,
// hand-written for gfx950 (MI355X).
//
// Method: paper digest "VC-Attention: Value Smoothing and Softmax Casting for
// Low-bit Attention", V-Smooth paragraph (the residual is quantised and each
// block mean is added back with one outer product of the row sums online
// softmax already keeps, without a second pass over V) and ExpCast-FP8 paragraph
// (the P byte is an affine function of the log-domain score: one fused
// multiply-add, round to nearest even, clip to the normal range, beta = -0.35).
// News article "Nunchux open-sources VC-Attention", sections "V-Smooth" (item
// Restore) and "ExpCast-FP8".
//
// Design (MI355X-first, not the pages' Blackwell kernel):
//  * one workgroup = 8 wavefronts = two 128-query blocks (one Q scale each)
//    sharing every K/V tile copy; every wavefront owns 32 queries and runs
//    V_MFMA_F32_32X32X64_F8F6F4 (OCP E4M3).
//  * scores are computed transposed, S^T = K . Q^T (K rows are the MFMA rows),
//    so each lane holds the scores of ONE query.  Row max needs one cross-lane
//    step, and the ExpCast bytes land directly in the lane layout of the
//    B operand of O^T = V^T . P^T: no shuffle of P.  The K rows of a tile are fed
//    to the MFMA in the order sigma() so that every lane's P bytes are 32
//    consecutive keys, matching 32 consecutive bytes of the transposed V block.
//  * K and V^T tiles (16 KiB each) are double-buffered in LDS with an XOR chunk
//    swizzle that keeps the 128-bit operand reads free of bank conflicts.
//  * the row sum of the decoded P bytes comes from a 16x16x128 FP8 MFMA against
//    a ones pattern (exact: every E4M3 value is a multiple of 2^-9), and the
//    block means are restored four blocks at a time, U += sum_t rowsum_t (x)
//    mean_t / sv, by one bf16 MFMA per 32 channels with each factor split into
//    a bf16 pair (relative error below 2^-16), so no VALU instruction touches
//    the accumulators except the (rare) rescale when a running max moves.  A
//    tile's row sum is consumed at the start of the next tile, so no wavefront
//    waits for its P.V MFMAs before the tile's barrier.
//  * tiles are copied global -> LDS through buffer resources, the next tile's
//    copies issued between the Q.K MFMAs (not all at the start of a tile, where
//    the eight wavefronts would queue behind each other in the address unit);
//    the Q block scale is scalar and the next K block scale is prefetched at
//    the start of the tile, so no wait for a copy sits inside a tile; the row
//    max crosses the two 32-lane halves with V_PERMLANE32_SWAP (no LDS).
//  * workgroups are ordered head-major and handed to the 8 XCDs in contiguous
//    ranges, so the workgroups sharing an XCD's L2 stream the same K/V blocks.
#include <type_traits>

#include "attn_common.h"

namespace vc {

constexpr int kAttnThreads = 512;   // 8 wavefronts: two 128-query blocks sharing each K/V tile
constexpr int kTile = kBlock * kD;   // bytes of one K or V^T tile

struct AttnArgs {
  const uint8_t* q;  const float* qs;
  const uint8_t* k;  const float* ks;
  const uint8_t* v;  const float* vs;
  const uint16_t* means;
  const uint8_t* vg;   // MXFP4: E8M0 group scales [BH][nb][128][2(g)][2(h)]
  float* out;
  float* sdump; uint8_t* pdump;
  int N, nb, BH;
  float c0;
};

// P.V with an MXFP4 V^T operand: A = 32 E2M1 values per lane (16 bytes, the
// upper half of the operand unused), B = P bytes (E4M3), the lane's E8M0 scale
// in byte H of `scale` (V_MFMA_SCALE_F32_32X32X64_F8F6F4, A format FP4).  Lane
// (row r, group g) holds keys 16g + [0, 16) and 32 + 16g + [0, 16) of the
// 64-key chunk against B lanes holding keys 32g + [0, 32): the instruction's
// operand layout, probed on the device.
template <int H>
__device__ __forceinline__ v16f mfma_pv_fp4(uint4 a4, const v8i& p, int scale, const v16f& c) {
  const v8i a = {(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, p, c, 4, 0, H, scale, 0, 127);
}

__device__ __forceinline__ v4f mfma16(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// max of a lane's value and that of lane l ^ 32, without LDS (V_PERMLANE32_SWAP)
__device__ __forceinline__ float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

// MFMA bursts run at raised wave priority, so a wavefront's MFMAs are issued
// as soon as the matrix unit frees up while the SIMD's other wavefront runs VALU
// work.
__device__ __forceinline__ void mfma_phase_begin() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void mfma_phase_end() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
}

template <int kPMode, bool kDump, int kVF>
__global__ void __launch_bounds__(kAttnThreads, 1) attn_fp8_e4m3(AttnArgs a) {
  constexpr bool kFP4 = kVF == VC_V_MXFP4;
  // V tile bytes in global memory: E4M3 128 x 128; MXFP4 128 channels x 64
  // bytes, then (in LDS only) the 512 bytes of E8M0 scales at offset 8192
  constexpr int kVTile = kFP4 ? kTile / 2 : kTile;
  // The two buffers of each operand are separate LDS objects so that reads of
  // one are not ordered behind the asynchronous copies into the other (the
  // copies are tracked by the vector memory counter).
  __shared__ __align__(16) uint8_t Ks0[kTile];
  __shared__ __align__(16) uint8_t Ks1[kTile];
  __shared__ __align__(16) uint8_t Vs0[kTile];
  __shared__ __align__(16) uint8_t Vs1[kTile];
  // A operands of the batched mean restore: per batch of four KV blocks, 16
  // bytes per (channel block cb, lane half g, column col): bf16 [hi, lo, hi, 0]
  // of mean_t / sv for channel 32 cb + col and blocks 2g, 2g + 1 of the batch.
  __shared__ __align__(16) uint32_t MuB[2][1024];
  __shared__ float InvSv[kD];
  __shared__ float Sv[kD];

  const int npair = (a.nb + 1) >> 1;
  const int item = xcd_item(blockIdx.x, npair * a.BH);
  const int bh = item / npair, pr = item % npair;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases stay scalar
  // wavefronts 4w..4w+3 take query block 2*pr + w; when nb is odd the last
  // pair's second block does not exist: it repeats the first and stores nothing
  const bool qvalid = 2 * pr + (wave >> 2) < a.nb;
  const int qb = qvalid ? 2 * pr + (wave >> 2) : 2 * pr;
  const int g = lane >> 5, col = lane & 31;
  const int N = a.N, nb = a.nb;
  const long long Np = (long long)nb * kBlock;

  if (tid < kD) {
    const float sv = a.vs[(long long)bh * kD + tid];
    const float svp = sv > 0.0f ? sv : 1.0f;   // an all-zero residual channel keeps its mean
    Sv[tid] = svp;
    InvSv[tid] = 1.0f / svp;
  }

  // Q operand (B of S^T = K.Q^T): query row, 32 bytes per channel half.
  const int qrow = qb * kBlock + (wave & 3) * 32 + col;
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
  // uniform: held in a scalar register, so no wait on it inside the tile loop
  const float sq = __builtin_bit_cast(
      float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, a.qs[(long long)bh * nb + qb])));

  const uint8_t* kbase = a.k + (long long)bh * Np * kD;
  const uint8_t* vbase = a.v + (long long)bh * nb * kVTile;
  const uint16_t* mbase = a.means + (long long)bh * nb * kD;

  // K and V^T tiles go global -> LDS directly.  Instruction j (16 per tile,
  // 4 per wave) fills LDS bytes [1024j, 1024j+1024): lane i writes row
  // 8j + i/8 at chunk position i%8, so it fetches the global chunk that the
  // XOR swizzle puts there.
  // The copies go through buffer resources (one head's nb tiles each), so the
  // tile offset is a scalar and a lane keeps only 32-bit in-tile offsets.
  // Rows of instructions i and i+2 differ by 64, which leaves swz_k unchanged,
  // and rows of any two differ by a multiple of 32, which leaves swz_v
  // unchanged: three lane offsets plus scalar offsets cover all eight copies.
  uint32_t mr = 0;
  float ksn = 0.0f;   // K scale of the block in flight; becomes the next block's
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, (uint32_t)nb * kTile);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, (uint32_t)nb * kVTile);
  // MXFP4 scales: 512 bytes per tile; lanes 32..63 of the copy read the next
  // tile's (or, past the end, zeros) into unused LDS bytes
  const __amdgpu_buffer_rsrc_t vgrs = make_rsrc(kFP4 ? a.vg + (long long)bh * nb * 512 : a.v, (uint32_t)nb * 512);
  uint32_t dkoff, dvoff;   // copy j = wave + 8i: rows of i = 0, 1 differ by 64 (neither swizzle changes)
  {
    const int pos = lane & 7;
    const int row = 8 * wave + (lane >> 3);
    dkoff = (uint32_t)(row * kD + 16 * (pos ^ swz_k(row)));
    dvoff = (uint32_t)(row * kD + 16 * (pos ^ swz_v(row)));
    if (kFP4) {   // one copy per wavefront: channel rows 16 wave .. 16 wave + 15, 4 chunks of 16 bytes each
      const int r4 = 16 * wave + (lane >> 2);
      dvoff = (uint32_t)(r4 * 64 + 16 * ((lane & 3) ^ ((r4 >> 2) & 3)));
    }
  }
  auto load_tile = [&](int t, int buf) {
    const uint32_t toff = (uint32_t)t * kTile;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int j = wave + 8 * i;
      dma16_buf(krs, (buf ? Ks1 : Ks0) + 1024 * j, dkoff, toff + 8192u * i);
      if (!kFP4) dma16_buf(vrs, (buf ? Vs1 : Vs0) + 1024 * j, dvoff, toff + 8192u * i);
    }
    if (kFP4) {
      dma16_buf(vrs, (buf ? Vs1 : Vs0) + 1024 * wave, dvoff, (uint32_t)t * kVTile);
      if (wave == 0) dma16_buf(vgrs, (buf ? Vs1 : Vs0) + 8192, (uint32_t)lane * 16u, (uint32_t)t * 512u);
    }
    if (tid < kD) mr = mbase[(long long)t * kD + tid];
    ksn = a.ks[(long long)bh * nb + t];   // K scale of the block being copied
  };
  // copy p (0..3) of tile t: E4M3 K half 0, V half 0, K half 1, V half 1;
  // MXFP4 K half 0, K half 1, V, E8M0 scales (wavefront 0).  Past the last tile
  // the buffer resources read zeros into a buffer that is not read again.
  auto copy_piece = [&](int t, int buf, int p) {
    const uint32_t toff = (uint32_t)t * kTile;
    if (!kFP4) {
      const int i = p >> 1, j = wave + 8 * i;
      if ((p & 1) == 0) dma16_buf(krs, (buf ? Ks1 : Ks0) + 1024 * j, dkoff, toff + 8192u * i);
      else dma16_buf(vrs, (buf ? Vs1 : Vs0) + 1024 * j, dvoff, toff + 8192u * i);
    } else if (p < 2) {
      dma16_buf(krs, (buf ? Ks1 : Ks0) + 1024 * (wave + 8 * p), dkoff, toff + 8192u * p);
    } else if (p == 2) {
      dma16_buf(vrs, (buf ? Vs1 : Vs0) + 1024 * wave, dvoff, (uint32_t)t * kVTile);
    } else if (wave == 0) {
      dma16_buf(vgrs, (buf ? Vs1 : Vs0) + 8192, (uint32_t)lane * 16u, (uint32_t)t * 512u);
    }
  };
  // mean_t / sv of tile t as a bf16 pair: hi = the value truncated to bf16
  // (exact difference), lo = the remainder rounded to bf16
  auto store_means = [&](int t) {
    if (tid < kD) {
      const float mu = bf16_bits_to_f32(mr) * InvSv[tid];
      const uint32_t hi = __float_as_uint(mu) & 0xFFFF0000u;
      const uint32_t lo = f32_to_bf16_rne(mu - __uint_as_float(hi));
      const int sl = t & 3;
      uint2 w;
      w.x = (hi >> 16) | (lo << 16);
      w.y = hi >> 16;
      *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(MuB[(t >> 2) & 1]) +
                                (((tid >> 5) * 2 + (sl >> 1)) * 32 + (tid & 31)) * 16 + 8 * (sl & 1)) = w;
    }
  };

  load_tile(0, 0);
  float ksc = ksn;
  // slots of blocks past the last one stay zero (0 x 0 in the final batch)
  reinterpret_cast<uint4*>(&MuB[0][0])[tid] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();          // InvSv ready
  store_means(0);
  wait_dma();
  __syncthreads();

  v16f o[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[cb][r] = 0.0f;
  float mx = -__builtin_inff();
  float l = 0.0f;
  // Row sums come from V_MFMA_F32_16X16X128_F8F6F4 with a P half (64 keys) as
  // the B operand: B lane l is column l%16 of k-group l/16, which holds query
  // l%32 over 32 of the half's keys.  A lane l (row l%16, k-group l/16) is E4M3
  // 1.0 when bit 2 of the row equals the parity of the k-group and 0 otherwise,
  // so output row r sums the two k-groups of query (r%8 < 4 ? col : col + 16).
  // Output lane l holds rows 4(l/16)..4(l/16)+3 of column l%16, which is the
  // row sum of query l%32: the lane's own query.
  v8i ones;
  {
    const int on = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) ones[i] = on ? 0x38383838 : 0;
  }
  // The mean restore is batched over four KV blocks: rsb[s] holds the row sum
  // of block s of the batch (rescaled with the accumulators while pending), and
  // one bf16 V_MFMA_F32_32X32X16_BF16 per 32-channel block adds
  // sum_s rsb[s] * mean_s / sv with each factor split into a bf16 pair
  // (hi*hi + lo*hi + hi*lo, three of the 16 k-slots per block; the dropped
  // lo*lo term and the rounding of lo are below 2^-16 of the product).
  float rsb[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  // The row sum of tile t is taken into l and rsb at the start of tile t + 1
  // (before that tile's rescale, so the arithmetic is unchanged): nothing waits
  // for the P.V MFMAs at the end of a tile, and they drain during the barrier.
  float rsp = 0.0f;
  // U += sum_s rsb[s] (x) mean_s / sv for the batch held in MuB[mbuf]: lanes of
  // half g carry blocks 2g, 2g + 1 as B k-slots [hi, hi, lo, 0] of each row sum
  auto restore = [&](int mbuf) {
    const float x0 = g ? rsb[2] : rsb[0];
    const float x1 = g ? rsb[3] : rsb[1];
    const uint32_t h0 = __float_as_uint(x0) & 0xFFFF0000u, h1 = __float_as_uint(x1) & 0xFFFF0000u;
    const uint4 bw = make_uint4(h0 | (h0 >> 16), f32_to_bf16_rne(x0 - __uint_as_float(h0)), h1 | (h1 >> 16),
                                f32_to_bf16_rne(x1 - __uint_as_float(h1)));
    const v8bf bop = __builtin_bit_cast(v8bf, bw);
    const uint8_t* mb = reinterpret_cast<const uint8_t*>(MuB[mbuf]) + (g * 32 + col) * 16;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
      o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(mb + 1024 * cb)), bop, o[cb], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) rsb[i] = 0.0f;
  };
  // LDS operand addresses: the K rows sigma(m, col) of the four 32-key blocks
  // differ by multiples of 16 rows and the V rows 32*cb + col by multiples of 32,
  // neither of which changes the swizzle, so four base offsets per operand plus
  // compile-time offsets cover every read.
  uint32_t lk[4], lv[4];
  {
    const int kr = sigma(0, col), ksw = swz_k(kr), vsw = swz_v(col);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 4 * (i >> 1) + 2 * g + (i & 1);    // chunks 2g, 2g+1, 4+2g, 5+2g
      lk[i] = (uint32_t)(kr * kD + 16 * (c ^ ksw));
      lv[i] = (uint32_t)(col * kD + 16 * (c ^ vsw));
    }
  }
  // MXFP4 V^T operand: channel row 32cb + col, chunk 2h + g, swizzled like the copy
  uint32_t lv4[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) lv4[h] = (uint32_t)(col * 64 + 16 * ((2 * h + g) ^ ((col >> 2) & 3)));
  auto ld16 = [](const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); };
  auto op8 = [](uint4 lo, uint4 hi) {
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
  };

  // one KV block; the LDS buffer index is a compile-time constant so every
  // LDS address is a base register plus an immediate offset
  auto step = [&](const int t, auto slotc) {
    constexpr int slot = decltype(slotc)::value;   // t % 4: block within the restore batch
    constexpr int buf = slot & 1;
    if (t + 1 < nb) {
      if (tid < kD) mr = mbase[(long long)(t + 1) * kD + tid];
      ksn = a.ks[(long long)bh * nb + t + 1];   // K scale of the block being copied
    }

    // ---- row sum of the previous tile; restore of the batch it completed ----
    if (slot != 0 || t > 0) {
      l += rsp;
      rsb[(slot + 3) & 3] = rsp;
    }
    // ---- S^T = K_t . Q^T : 4 blocks of 32 keys x 32 queries ----
    mfma_phase_begin();
    if (slot == 0 && t > 0) restore(((t >> 2) - 1) & 1);
    v16f s[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[m][r] = 0.0f;
      const uint8_t* kb = (buf ? Ks1 : Ks0) + kD * (64 * (m >> 1) + 16 * (m & 1));
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
        s[m] = mfma32(op8(ld16(kb + lk[2 * c2]), ld16(kb + lk[2 * c2 + 1])), qop[c2], s[m]);
      // the next tile's copies, one per pair of Q.K MFMAs, so that they drain
      // through the address unit while the MFMAs run
      copy_piece(t + 1, buf ^ 1, m);
    }
    mfma_phase_end();
    // keys beyond N (last tile only) take no part
    if ((t + 1) * kBlock > N) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 64 * (m >> 1) + 32 * g + 16 * (m & 1) + r;
          if (t * kBlock + key >= N) s[m][r] = -__builtin_inff();
        }
    }
    // ---- running max (log2 units) ----
    float M = s[0][0];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) M = fmaxf(M, s[m][r]);
    M = max_across_halves(M);
    const float kap = (sq * ksc) * a.c0;
    const float mx_new = fmaxf(mx, M * kap);

    // ---- P bytes, laid out as the B operand of the P.V MFMA ----
    uint32_t pk[16];
    if (kPMode == VC_P_EXPCAST) {
      const float A = 8.0f * kap;
      const float Bc = 55.65f - 8.0f * mx_new;
      // codes never exceed 56 unless rounding of a huge running max pushes the
      // row maximum past 56.5; then clamp (the oracle clamps at 56 as well)
      if (__builtin_expect(__any(__builtin_fmaf(M, A, Bc) >= 56.5f), 0)) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[m][r] = fminf(s[m][r], (56.0f - Bc) / A);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t wv[4];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          uint32_t w = 0u;
#pragma unroll
          for (int b = 0; b < 4; ++b)   // round to nearest even, clamp to [0,255], pack
            w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s[m][4 * r4 + b], A, Bc), b, w);
          wv[r4] = w;
        }
        // flush codes 1..7 (below the E4M3 normal range) to 0, eight bytes at a
        // time: codes are <= 56, so adding 0x78 to every byte carries nowhere and
        // sets a byte's top bit exactly when its code is >= 8; V_PERM_B32 spreads
        // those top bits (bytes 1, 3 directly, bytes 0, 2 from the copy shifted
        // left by 8) into byte masks.
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const uint64_t w64 = ((uint64_t)wv[2 * pr + 1] << 32) | wv[2 * pr];
          const uint64_t t = w64 + 0x7878787878787878ull;
          const uint64_t t8 = t << 8;
          pk[4 * m + 2 * pr] = wv[2 * pr] & __builtin_amdgcn_perm((uint32_t)t8, (uint32_t)t, 0x090B080Au);
          pk[4 * m + 2 * pr + 1] =
              wv[2 * pr + 1] & __builtin_amdgcn_perm((uint32_t)(t8 >> 32), (uint32_t)(t >> 32), 0x090B080Au);
        }
      }
    } else {   // VC_P_FP32EXP_E4M3: conventional exp2 then E4M3 conversion
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          float p[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) p[b] = __builtin_amdgcn_exp2f(s[m][4 * r4 + b] * kap - mx_new);
          pk[4 * m + r4] = __builtin_amdgcn_cvt_pk_fp8_f32(
              p[2], p[3], __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0u, false), true);
        }
    }

    // keys at or beyond N (last tile only): P byte 0.  Their scores were set
    // to -inf for the row max, and -inf * kap is NaN when kap = 0 (an all-zero
    // Q block or K block has scale 0), so the bytes are cleared after the fact.
    if ((t + 1) * kBlock > N) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int key0 = t * kBlock + 64 * (m >> 1) + 32 * g + 16 * (m & 1) + 4 * r4;
          const int nv = min(max(N - key0, 0), 4);   // valid keys among the four bytes
          pk[4 * m + r4] &= nv >= 4 ? 0xFFFFFFFFu : (1u << (8 * nv)) - 1u;
        }
    }

    if (kDump && qvalid && qrow < N) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 64 * (m >> 1) + 32 * g + 16 * (m & 1) + r;
          const long long idx = ((long long)bh * N + qrow) * Np + (long long)t * kBlock + key;
          const bool valid = t * kBlock + key < N;
          a.sdump[idx] = valid ? s[m][r] : 0.0f;
          a.pdump[idx] = (uint8_t)(valid ? (pk[4 * m + (r >> 2)] >> (8 * (r & 3))) & 0xFFu : 0u);
        }
    }

    // ---- rescale the accumulators when the running max moved ----
    const float alpha = __builtin_amdgcn_exp2f(mx - mx_new);
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[cb][r] *= alpha;
#pragma unroll
      for (int i = 0; i < slot; ++i) rsb[i] *= alpha;
    }
    l *= alpha;
    mx = mx_new;

    // ---- O^T += V^T_t . P^T ; row sums from an all-ones operand ----
    mfma_phase_begin();
    v4f rs = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v8i pop;
#pragma unroll
      for (int i = 0; i < 8; ++i) pop[i] = (int)pk[8 * h + i];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        if constexpr (kFP4) {
          const uint8_t* vb = (buf ? Vs1 : Vs0) + 64 * 32 * cb;
          const int sc = (int)*reinterpret_cast<const uint16_t*>((buf ? Vs1 : Vs0) + 8192 + (32 * cb + col) * 4 + 2 * g);
          o[cb] = h == 0 ? mfma_pv_fp4<0>(ld16(vb + lv4[0]), pop, sc, o[cb])
                         : mfma_pv_fp4<1>(ld16(vb + lv4[1]), pop, sc, o[cb]);
        } else {
          const uint8_t* vb = (buf ? Vs1 : Vs0) + kD * 32 * cb;
          o[cb] = mfma32(op8(ld16(vb + lv[2 * h]), ld16(vb + lv[2 * h + 1])), pop, o[cb]);
        }
      }
      rs = mfma16(ones, pop, rs);
    }
    rsp = rs[0];   // taken into l and rsb at the start of the next tile
    mfma_phase_end();

    if (t + 1 < nb) store_means(t + 1);
    wait_dma();
    __syncthreads();
    ksc = ksn;
  };

  for (int t = 0; t < nb; t += 4) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < nb) step(t + 1, std::integral_constant<int, 1>{});
    if (t + 2 < nb) step(t + 2, std::integral_constant<int, 2>{});
    if (t + 3 < nb) step(t + 3, std::integral_constant<int, 3>{});
  }
  // the last tile's row sum and the restore of the final (possibly partial) batch
  l += rsp;
  {
    const int sl = (nb - 1) & 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) rsb[i] = i == sl ? rsp : rsb[i];
  }
  restore(((nb - 1) >> 2) & 1);

  // ---- epilogue: O = sv * U / l, original query order ----
  if (qvalid && qrow < N) {
    const float invl = 1.0f / l;
    float* op = a.out + ((long long)bh * N + qrow) * kD;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int c0 = 32 * cb + 8 * a4 + 4 * g;
        float4 val;
        val.x = o[cb][4 * a4 + 0] * Sv[c0 + 0] * invl;
        val.y = o[cb][4 * a4 + 1] * Sv[c0 + 1] * invl;
        val.z = o[cb][4 * a4 + 2] * Sv[c0 + 2] * invl;
        val.w = o[cb][4 * a4 + 3] * Sv[c0 + 3] * invl;
        *reinterpret_cast<float4*>(op + c0) = val;
      }
  }
}

template <int kPMode, bool kDump, int kVF>
static void launch_one(const AttnArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(((a.nb + 1) / 2) * a.BH));   // one workgroup per pair of query blocks
  hipLaunchKernelGGL((attn_fp8_e4m3<kPMode, kDump, kVF>), grid, dim3(kAttnThreads), 0, st, a);
}

template <int kPMode, int kVF>
static void launch_pm(const AttnArgs& a, bool dump, hipStream_t st) {
  if (dump) launch_one<kPMode, true, kVF>(a, st);
  else launch_one<kPMode, false, kVF>(a, st);
}

static int launch_e4m3(const AttnArgs& a, int p_mode, bool dump, hipStream_t st, bool fp4 = false) {
  if (fp4) {
    if (p_mode == VC_P_EXPCAST) launch_pm<VC_P_EXPCAST, VC_V_MXFP4>(a, dump, st);
    else launch_pm<VC_P_FP32EXP_E4M3, VC_V_MXFP4>(a, dump, st);
  } else {
    if (p_mode == VC_P_EXPCAST) launch_pm<VC_P_EXPCAST, VC_V_E4M3>(a, dump, st);
    else launch_pm<VC_P_FP32EXP_E4M3, VC_V_E4M3>(a, dump, st);
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? VC_OK : vc_set_hip_error((int)e);
}

float score_scale_c0(float softmax_scale) {  // c0 = fp32(scale * log2 e)
  return (float)((double)softmax_scale * 1.4426950408889634);
}

}  // namespace vc

using namespace vc;

int vc_attn_nvfp4_launch(const uint8_t* q_codes, const float* q_scales, const uint8_t* k_codes,
                         const float* k_scales, const uint8_t* v_codes, const float* v_scales,
                         const uint8_t* v_group_scales, const uint16_t* v_means, int B, int H, int N,
                         float c0, float* out, float* s_dump, uint16_t* p_dump, hipStream_t st);

extern "C" int vc_attn_fp8_fwd(const uint8_t* q_codes, const float* q_scales, const uint8_t* k_codes,
                               const float* k_scales, const uint8_t* v_codes, const float* v_scales,
                               const uint8_t* v_group_scales, const uint16_t* v_means, int B, int H, int N,
                               int d, float softmax_scale, int p_mode, int v_format, float* out,
                               void* stream) {
  if (d != kD) return VC_ERR_UNSUPPORTED;
  if (!q_codes || !q_scales || !k_codes || !k_scales || !v_codes || !v_scales || !v_means || !out)
    return VC_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return VC_ERR_INVALID_ARG;
  const int nb = (N + kBlock - 1) / kBlock;
  if ((long long)nb * B * H > 0x7FFFFFFFLL) return VC_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float c0 = score_scale_c0(softmax_scale);
  if (v_format == VC_V_E4M3 && (p_mode == VC_P_EXPCAST || p_mode == VC_P_FP32EXP_E4M3)) {
    AttnArgs a{q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, v_means, nullptr, out, nullptr, nullptr,
               N, nb, B * H, c0};
    return launch_e4m3(a, p_mode, false, st);
  }
  if (v_format == VC_V_MXFP4 && (p_mode == VC_P_EXPCAST || p_mode == VC_P_FP32EXP_E4M3)) {
    if (!v_group_scales) return VC_ERR_INVALID_ARG;
    AttnArgs a{q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, v_means, v_group_scales, out, nullptr,
               nullptr, N, nb, B * H, c0};
    return launch_e4m3(a, p_mode, false, st, true);
  }
  if (v_format == VC_V_NVFP4 && p_mode == VC_P_FP32_BF16) {
    if (!v_group_scales) return VC_ERR_INVALID_ARG;
    return vc_attn_nvfp4_launch(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, v_group_scales,
                                v_means, B, H, N, c0, out, nullptr, nullptr, st);
  }
  return VC_ERR_UNSUPPORTED;
}

extern "C" int vc_attn_fwd_dump(const uint8_t* q_codes, const float* q_scales, const uint8_t* k_codes,
                                const float* k_scales, const uint8_t* v_codes, const float* v_scales,
                                const uint8_t* v_group_scales, const uint16_t* v_means, int B, int H, int N, int d,
                                float softmax_scale, int p_mode, int v_format, float* out, float* s_dump,
                                void* p_dump, void* stream) {
  if (d != kD) return VC_ERR_UNSUPPORTED;
  if (!q_codes || !q_scales || !k_codes || !k_scales || !v_codes || !v_scales || !v_means || !out || !s_dump ||
      !p_dump)
    return VC_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return VC_ERR_INVALID_ARG;
  const int nb = (N + kBlock - 1) / kBlock;
  if ((long long)nb * B * H > 0x7FFFFFFFLL) return VC_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float c0 = score_scale_c0(softmax_scale);
  const bool e4m3_p = p_mode == VC_P_EXPCAST || p_mode == VC_P_FP32EXP_E4M3;
  if ((v_format == VC_V_E4M3 || v_format == VC_V_MXFP4) && e4m3_p) {
    if (v_format == VC_V_MXFP4 && !v_group_scales) return VC_ERR_INVALID_ARG;
    AttnArgs a{q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, v_means,
               v_format == VC_V_MXFP4 ? v_group_scales : nullptr, out, s_dump, static_cast<uint8_t*>(p_dump),
               N, nb, B * H, c0};
    return launch_e4m3(a, p_mode, true, st, v_format == VC_V_MXFP4);
  }
  if (v_format == VC_V_NVFP4 && p_mode == VC_P_FP32_BF16) {
    if (!v_group_scales) return VC_ERR_INVALID_ARG;
    return vc_attn_nvfp4_launch(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, v_group_scales,
                                v_means, B, H, N, c0, out, s_dump, static_cast<uint16_t*>(p_dump), st);
  }
  return VC_ERR_UNSUPPORTED;
}

extern "C" int vc_attn_fp8_fwd_dump(const uint8_t* q_codes, const float* q_scales, const uint8_t* k_codes,
                                    const float* k_scales, const uint8_t* v_codes, const float* v_scales,
                                    const uint16_t* v_means, int B, int H, int N, int d, float softmax_scale,
                                    int p_mode, float* out, float* s_dump, uint8_t* p_dump, void* stream) {
  if (p_mode != VC_P_EXPCAST && p_mode != VC_P_FP32EXP_E4M3) return VC_ERR_UNSUPPORTED;
  return vc_attn_fwd_dump(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, nullptr, v_means, B, H, N, d,
                          softmax_scale, p_mode, VC_V_E4M3, out, s_dump, p_dump, stream);
}
