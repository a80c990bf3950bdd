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
//    the accumulators except the rescale when a running max moves.
//  * software pipeline inside each wavefront: the Q.K MFMAs of tile t run
//    beside the flush of tile t-1's P bytes and tile t's block maxima; tile t's
//    ExpCast bytes (one fmaf + one byte conversion per score) run beside the
//    P.V and row-sum MFMAs of tile t-1.  V is copied one tile behind K, so two
//    LDS buffers of each suffice; operand reads run two MFMAs ahead; the
//    rescale of the accumulators is deferred one step so that it never waits
//    for MFMAs still in flight.
//  * tiles are copied global -> LDS through buffer resources, issued between
//    the Q.K MFMAs; the Q block scale is scalar and the next K block scale is
//    prefetched at the start of the tile, so no wait for a copy sits inside a
//    tile; the row max crosses the two 32-lane halves with V_PERMLANE32_SWAP.
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

// The kernel is software-pipelined inside every wavefront so that each MFMA
// burst has independent VALU work beside it:
//   stage 1 of tile t: the Q.K MFMAs of tile t, beside them the flush of tile
//            t-1's P bytes (codes 1..7 -> 0) and the row max of tile t;
//   stage 2 of tile t: the ExpCast bytes of tile t (one fmaf + one byte
//            conversion per score), beside them the P.V and row-sum MFMAs of
//            tile t-1.
// V is copied one tile behind K (V of tile t during tile t, K of tile t+1
// during tile t), so two buffers of each still suffice.  The accumulators see
// the same sequence as in the unpipelined order: P.V of tile t-1 is added in
// the scale of the running max after tile t-1, then the rescale to tile t's
// max.  A tile's row sum is taken into l (times the rescale that followed it)
// at the start of the next tile, and a batch of four row sums is restored in
// the tile after that, so no wavefront waits for an MFMA result.
template <int kPMode, bool kDump, int kVF>
__global__ void __launch_bounds__(kAttnThreads, 1) attn_fp8_e4m3(AttnArgs a) {
  constexpr bool kFP4 = kVF == VC_V_MXFP4;
  constexpr int kVTile = kFP4 ? kTile / 2 : kTile;
  __shared__ __align__(16) uint8_t Ks0[kTile];
  __shared__ __align__(16) uint8_t Ks1[kTile];
  __shared__ __align__(16) uint8_t Vs0[kTile];
  __shared__ __align__(16) uint8_t Vs1[kTile];
  __shared__ __align__(16) uint32_t MuB[2][1024];
  __shared__ float InvSv[kD];
  __shared__ float Sv[kD];

  const int npair = (a.nb + 1) >> 1;
  const int item = xcd_item(blockIdx.x, npair * a.BH);
  const int bh = item / npair, pr = item % npair;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool qvalid = 2 * pr + (wave >> 2) < a.nb;
  const int qb = qvalid ? 2 * pr + (wave >> 2) : 2 * pr;
  const int g = lane >> 5, col = lane & 31;
  const int N = a.N, nb = a.nb;
  const long long Np = (long long)nb * kBlock;

  if (tid < kD) {
    const float sv = a.vs[(long long)bh * kD + tid];
    const float svp = sv > 0.0f ? sv : 1.0f;
    Sv[tid] = svp;
    InvSv[tid] = 1.0f / svp;
  }
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
  const float sq = __builtin_bit_cast(
      float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, a.qs[(long long)bh * nb + qb])));

  const uint8_t* kbase = a.k + (long long)bh * Np * kD;
  const uint8_t* vbase = a.v + (long long)bh * nb * kVTile;
  const uint16_t* mbase = a.means + (long long)bh * nb * kD;
  uint32_t mr = 0;
  float ksn = 0.0f;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, (uint32_t)nb * kTile);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, (uint32_t)nb * kVTile);
  const __amdgpu_buffer_rsrc_t vgrs = make_rsrc(kFP4 ? a.vg + (long long)bh * nb * 512 : a.v, (uint32_t)nb * 512);
  uint32_t dkoff, dvoff;
  {
    const int pos = lane & 7;
    const int row = 8 * wave + (lane >> 3);
    dkoff = (uint32_t)(row * kD + 16 * (pos ^ swz_k(row)));
    dvoff = (uint32_t)(row * kD + 16 * (pos ^ swz_v(row)));
    if (kFP4) {
      const int r4 = 16 * wave + (lane >> 2);
      dvoff = (uint32_t)(r4 * 64 + 16 * ((lane & 3) ^ ((r4 >> 2) & 3)));
    }
  }
  // half i (0, 1) of K tile t into buffer buf.  The last step asks for tile nb,
  // which does not exist: it copies tile nb - 1 again into a buffer that is not
  // read again (the buffer's scalar offset is outside the record-count check,
  // so it never points past the head's codes)
  auto copy_k = [&](int t, int buf, int i) {
    dma16_buf(krs, (buf ? Ks1 : Ks0) + 1024 * (wave + 8 * i), dkoff, (uint32_t)min(t, nb - 1) * kTile + 8192u * i);
  };
  // piece i (0, 1) of V tile t (t < nb) into buffer buf: E4M3 the two halves;
  // MXFP4 the codes, then the E8M0 scales (wavefront 0)
  auto copy_v = [&](int t, int buf, int i) {
    if (!kFP4) dma16_buf(vrs, (buf ? Vs1 : Vs0) + 1024 * (wave + 8 * i), dvoff, (uint32_t)t * kTile + 8192u * i);
    else if (i == 0) dma16_buf(vrs, (buf ? Vs1 : Vs0) + 1024 * wave, dvoff, (uint32_t)t * kVTile);
    else if (wave == 0) dma16_buf(vgrs, (buf ? Vs1 : Vs0) + 8192, (uint32_t)lane * 16u, (uint32_t)t * 512u);
  };
  // the block means of restore batch j (tiles 4j .. 4j+3): thread tid takes
  // channel tid % 128 of tile 4j + tid / 128 (tiles past the last one reload it:
  // their row sums are zero)
  auto load_means = [&](int j) {
    mr = mbase[(long long)min(4 * j + (tid >> 7), nb - 1) * kD + (tid & (kD - 1))];
  };
  auto store_means = [&](int j) {
    const int c = tid & (kD - 1), sl = tid >> 7;
    const float mu = bf16_bits_to_f32(mr) * InvSv[c];
    const uint32_t hi = __float_as_uint(mu) & 0xFFFF0000u;
    const uint32_t lo = f32_to_bf16_rne(mu - __uint_as_float(hi));
    uint2 w;
    w.x = (hi >> 16) | (lo << 16);
    w.y = hi >> 16;
    *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(MuB[j & 1]) +
                              (((c >> 5) * 2 + (sl >> 1)) * 32 + (c & 31)) * 16 + 8 * (sl & 1)) = w;
  };

  copy_k(0, 0, 0);
  copy_k(0, 0, 1);
  load_means(0);
  ksn = a.ks[(long long)bh * nb];
  float ksc = ksn;
  reinterpret_cast<uint4*>(&MuB[0][0])[tid] = make_uint4(0u, 0u, 0u, 0u);
  // V buffer 1 holds no tile before tile 1's copy: zeros, so that the (all-zero)
  // P.V of "tile -1" in the first step reads finite values
  reinterpret_cast<uint4*>(Vs1)[tid] = make_uint4(0u, 0u, 0u, 0u);
  reinterpret_cast<uint4*>(Vs1)[tid + kAttnThreads] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
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
  v8i ones;
  {
    const int on = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) ones[i] = on ? 0x38383838 : 0;
  }
  float rsb[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  v4f rsacc = {0.0f, 0.0f, 0.0f, 0.0f};   // row sum of the tile whose P.V ran last (pending)
  float alpha_prev = 1.0f;                 // rescale applied after that P.V
  uint32_t pk[16];                         // P bytes of the previous tile (pending flush and P.V)
#pragma unroll
  for (int i = 0; i < 16; ++i) pk[i] = 0u;

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
  // the pending row sum (times the rescale after it) joins l and slot sl of the batch
  auto take_rowsum = [&](int sl) {
    const float rv = rsacc[0] * alpha_prev;
    l += rv;
#pragma unroll
    for (int i = 0; i < 4; ++i) rsb[i] = i == sl ? rv : rsb[i];
  };
  uint32_t lk[4], lv[4];
  {
    const int kr = sigma(0, col), ksw = swz_k(kr), vsw = swz_v(col);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 4 * (i >> 1) + 2 * g + (i & 1);
      lk[i] = (uint32_t)(kr * kD + 16 * (c ^ ksw));
      lv[i] = (uint32_t)(col * kD + 16 * (c ^ vsw));
    }
  }
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
  // flush codes 1..7 of the pending P bytes to 0, eight bytes at a time: codes
  // are <= 56, so adding 0x78 to every byte carries nowhere and sets a byte's
  // top bit exactly when its code is >= 8; V_PERM_B32 spreads those top bits
  // (bytes 1, 3 directly, bytes 0, 2 from the copy shifted left by 8) into byte masks
  auto flush_q = [&](int q) {
    const uint64_t w64 = ((uint64_t)pk[2 * q + 1] << 32) | pk[2 * q];
    const uint64_t t = w64 + 0x7878787878787878ull;
    const uint64_t t8 = t << 8;
    pk[2 * q] &= __builtin_amdgcn_perm((uint32_t)t8, (uint32_t)t, 0x090B080Au);
    pk[2 * q + 1] &= __builtin_amdgcn_perm((uint32_t)(t8 >> 32), (uint32_t)(t >> 32), 0x090B080Au);
  };
  auto flush = [&]() {
#pragma unroll
    for (int q = 0; q < 8; ++q) flush_q(q);
  };
  // keys at or beyond N of tile t (the last): P byte 0 whatever the score scale
  auto mask_pk = [&](int t) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int key0 = t * kBlock + 64 * (m >> 1) + 32 * g + 16 * (m & 1) + 4 * r4;
        const int nv = min(max(N - key0, 0), 4);
        pk[4 * m + r4] &= nv >= 4 ? 0xFFFFFFFFu : (1u << (8 * nv)) - 1u;
      }
  };
  auto dump_p = [&](int t) {
    if (kDump && qvalid && qrow < N) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 64 * (m >> 1) + 32 * g + 16 * (m & 1) + r;
          const long long idx = ((long long)bh * N + qrow) * Np + (long long)t * kBlock + key;
          a.pdump[idx] = (uint8_t)(t * kBlock + key < N ? (pk[4 * m + (r >> 2)] >> (8 * (r & 3))) & 0xFFu : 0u);
        }
    }
  };
  // O^T += V^T . P^T for the pending P bytes (V tile in buffer vb), and their row sums
  auto pv = [&](auto vbc) {
    constexpr int vbuf = decltype(vbc)::value;
    v4f rs = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v8i pop;
#pragma unroll
      for (int i = 0; i < 8; ++i) pop[i] = (int)pk[8 * h + i];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        if constexpr (kFP4) {
          const uint8_t* vb = (vbuf ? Vs1 : Vs0) + 64 * 32 * cb;
          const int sc = (int)*reinterpret_cast<const uint16_t*>((vbuf ? Vs1 : Vs0) + 8192 + (32 * cb + col) * 4 + 2 * g);
          o[cb] = h == 0 ? mfma_pv_fp4<0>(ld16(vb + lv4[0]), pop, sc, o[cb])
                         : mfma_pv_fp4<1>(ld16(vb + lv4[1]), pop, sc, o[cb]);
        } else {
          const uint8_t* vb = (vbuf ? Vs1 : Vs0) + kD * 32 * cb;
          o[cb] = mfma32(op8(ld16(vb + lv[2 * h]), ld16(vb + lv[2 * h + 1])), pop, o[cb]);
        }
      }
      rs = mfma16(ones, pop, rs);
    }
    rsacc = rs;
  };

  // one KV tile (slot = t % 4, compile-time).  The MFMA bursts and the VALU
  // work beside them share one basic block: in the first steps the pending
  // row sum, P bytes and restore batch are zeros, so no step branches on t.
  auto step = [&](const int t, auto slotc) {
    constexpr int slot = decltype(slotc)::value;
    constexpr int cur = slot & 1;   // buffers of K tile t and V tile t; V tile t-1 is in cur ^ 1
    {
      const int tn = min(t + 1, nb - 1);   // next block (the last step reloads its own, unused)
      ksn = a.ks[(long long)bh * nb + tn];
      // the means of the next restore batch: loaded in slot 0, paired in slot 2
      // (after the restore of slot 1 has read the buffer they overwrite)
      if (slot == 0) load_means((t >> 2) + 1);
    }
    // ---- the row sum of tile t-2 joins l ----
    take_rowsum((slot + 2) & 3);

    // ---- stage 1: S^T = K_t . Q^T in four chunks, one 32-key block each; beside
    // a chunk's two MFMAs run the operand reads of the next chunk, a quarter of
    // the flush of tile t-1's P bytes and the maximum of the previous block
    // (whose MFMAs are two behind), each fixed in place so that the optimiser
    // neither sinks the maxima past the MFMAs nor the flush into stage 2 ----
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* kt = cur ? Ks1 : Ks0;
    auto kread = [&](int m, int c2) {
      const uint8_t* kb = kt + kD * (64 * (m >> 1) + 16 * (m & 1));
      return op8(ld16(kb + lk[2 * c2]), ld16(kb + lk[2 * c2 + 1]));
    };
    v16f s[4];
    float Mb[4];
    v8i ka = kread(0, 0), kc = kread(0, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v8i na = ka, nc = kc;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[m][r] = 0.0f;
      s[m] = mfma32(ka, qop[0], s[m]);
      if (m < 3) na = kread(m + 1, 0);
      if (kPMode == VC_P_EXPCAST) {
        flush_q(2 * m);
        asm volatile("" : "+v"(pk[4 * m]), "+v"(pk[4 * m + 1]));
      }
      s[m] = mfma32(kc, qop[1], s[m]);
      if (m < 3) nc = kread(m + 1, 1);
      if (kPMode == VC_P_EXPCAST) {
        flush_q(2 * m + 1);
        asm volatile("" : "+v"(pk[4 * m + 2]), "+v"(pk[4 * m + 3]));
      }
      if ((m & 1) == 0) copy_k(t + 1, cur ^ 1, m >> 1);
      else copy_v(t, cur, m >> 1);
      if (m >= 1) {
        Mb[m - 1] = s[m - 1][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) Mb[m - 1] = fmaxf(Mb[m - 1], s[m - 1][r]);
        asm volatile("" : "+v"(Mb[m - 1]));
      }
      __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);   // flush share
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA 2m
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // reads for MFMA 2m + 2
      __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);   // flush share
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA 2m + 1
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // reads for MFMA 2m + 3
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // tile copy
      __builtin_amdgcn_sched_group_barrier(0x002, 9, 0);   // block maximum
      __builtin_amdgcn_sched_barrier(0);
      ka = na;
      kc = nc;
    }
    {   // block 3 ends the Q.K MFMAs: a tree keeps its maximum's dependent chain short
      float u[6];
#pragma unroll
      for (int j = 0; j < 5; ++j) u[j] = fmaxf(fmaxf(s[3][3 * j], s[3][3 * j + 1]), s[3][3 * j + 2]);
      u[5] = s[3][15];
      Mb[3] = fmaxf(fmaxf(fmaxf(u[0], u[1]), u[2]), fmaxf(fmaxf(u[3], u[4]), u[5]));
    }
    float M = fmaxf(fmaxf(Mb[0], Mb[1]), fmaxf(Mb[2], Mb[3]));
    if ((t + 1) * kBlock > N) {   // last tile: keys beyond N take no part
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 64 * (m >> 1) + 32 * g + 16 * (m & 1) + r;
          if (t * kBlock + key >= N) s[m][r] = -__builtin_inff();
        }
      M = s[0][0];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) M = fmaxf(M, s[m][r]);
    }
    if (t > 0) dump_p(t - 1);
    if (kDump && qvalid && qrow < N) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 64 * (m >> 1) + 32 * g + 16 * (m & 1) + r;
          const long long idx = ((long long)bh * N + qrow) * Np + (long long)t * kBlock + key;
          a.sdump[idx] = t * kBlock + key < N ? s[m][r] : 0.0f;
        }
    }
    M = max_across_halves(M);
    const float kap = (sq * ksc) * a.c0;
    const float mx_new = fmaxf(mx, M * kap);

    // ---- the rescale to tile t-1's max, deferred from the previous step so that
    // it never waits for the P.V MFMAs just issued; then a completed batch of
    // four row sums is restored (accumulators and row sums in the same scale) ----
    if (__any(alpha_prev != 1.0f)) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[cb][r] *= alpha_prev;
    }
    if (slot == 1) restore(((t - 2) >> 2) & 1);

    // ---- stage 2: P bytes of tile t; beside them P.V and row sums of tile t-1 ----
    uint32_t pn[16];
    __builtin_amdgcn_sched_barrier(0);
    if (kPMode == VC_P_EXPCAST) {
      const float A = 8.0f * kap;
      const float Bc = 55.65f - 8.0f * mx_new;
      if (__builtin_expect(__any(__builtin_fmaf(M, A, Bc) >= 56.5f), 0)) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[m][r] = fminf(s[m][r], (56.0f - Bc) / A);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          uint32_t w = 0u;
#pragma unroll
          for (int b = 0; b < 4; ++b)
            w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s[m][4 * r4 + b], A, Bc), b, w);
          pn[4 * m + r4] = w;
        }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          float p[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) p[b] = __builtin_amdgcn_exp2f(s[m][4 * r4 + b] * kap - mx_new);
          pn[4 * m + r4] = __builtin_amdgcn_cvt_pk_fp8_f32(
              p[2], p[3], __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0u, false), true);
        }
    }
    pv(std::integral_constant<int, cur ^ 1>{});
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(pn[i]));
    // issue order: operand reads two P.V MFMAs ahead; a share of the P bytes of
    // tile t under the first reads' latency, then one after each of the ten
    // MFMAs (eight P.V, two row sums)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 13, 0);
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kPMode == VC_P_EXPCAST ? 13 : 22, 0);
      if (i < 6) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- rescale to tile t's max: l and the pending row sums now, the
    // accumulators (which tile t-1's P.V MFMAs are still writing) next step ----
    const float alpha = __builtin_amdgcn_exp2f(mx - mx_new);
#pragma unroll
    for (int i = 0; i < 4; ++i) rsb[i] *= alpha;
    l *= alpha;
    alpha_prev = alpha;
    mx = mx_new;
#pragma unroll
    for (int i = 0; i < 16; ++i) pk[i] = pn[i];

    if (slot == 2) store_means((t >> 2) + 1);
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
  // ---- drain: row sum of tile nb-2, P.V and row sum of tile nb-1, last restores ----
  if (nb >= 2) take_rowsum((nb - 2) & 3);
  if (__any(alpha_prev != 1.0f)) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[cb][r] *= alpha_prev;
  }
  if (nb >= 2 && ((nb - 2) & 3) == 3) restore(((nb - 2) >> 2) & 1);
  if (kPMode == VC_P_EXPCAST) flush();
  mask_pk(nb - 1);
  dump_p(nb - 1);
  if ((nb - 1) & 1) pv(std::integral_constant<int, 1>{});
  else pv(std::integral_constant<int, 0>{});
  alpha_prev = 1.0f;
  take_rowsum((nb - 1) & 3);
  restore(((nb - 1) >> 2) & 1);

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
  if ((long long)nb * kTile > 0xFFFFFFFFLL) return VC_ERR_INVALID_ARG;   // a head's codes in one buffer record
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
  if ((long long)nb * kTile > 0xFFFFFFFFLL) return VC_ERR_INVALID_ARG;   // a head's codes in one buffer record
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
