// V-Smooth grouping on gfx950: k-means over the Value tokens of every
// (batch, head) and a stable sort of the tokens by cluster label.
//
// Method: paper digest "VC-Attention: Value Smoothing and Softmax Casting for
// Low-bit Attention", V-Smooth paragraph (online k-means per batch and head,
// Key and Value reordered by cluster label); news article "Nunchux open-sources
// VC-Attention", section "V-Smooth", item Group.
//
// The arithmetic is fixed so that labels are reproducible bit for bit:
//   distance  dot = fmaf chain over channels 0..127, cc = same for c.c,
//             score = fmaf(-2, dot, cc); argmin, lowest index on ties
//   update    int64 sums of rint(v * 2^24) (order-free, so atomics are exact),
//             centroid = (float)((double)sum * 2^-24 / (double)count)
//
// Kernels (all on the caller's stream, launched T times for assign/update):
//   kmeans_init         centroid c <- V[floor(c*N/k)], zero the sums, |c|^2
//   kmeans_assign_mfma  labels and counts for k <= 64: an int8 MFMA screen with a
//                       rigorous bound, the fixed-order rule for open tokens
//   kmeans_assign       labels and counts for k > 64: one token per lane, four
//                       independent FMA chains (centroids through the scalar
//                       cache: uniform addresses)
//   kmeans_accum        fixed-point sums: tokens one at a time, lanes over
//                       channels, into LDS (k <= 64; conflict-free), then one
//                       global atomic per non-zero partial of the 4096-token
//                       block; after the first pass only tokens whose label moved
//   kmeans_update       new centroids from the persistent sums, zero the counts, |c|^2
//   sort_hist / sort_scan / sort_scatter   stable counting sort by label
#include <type_traits>

#include "vc_common.h"

namespace vc {

constexpr int kAssignThreads = 256;
constexpr int kTokPerThread = 2;
constexpr int kTokPerWG = kAssignThreads * kTokPerThread;  // 512 tokens
constexpr int kAccThreads = 1024;
constexpr int kMTokWG = 2048;                              // tokens per screened-assignment workgroup
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr int kAccTok = 4096;                              // tokens per accumulation workgroup
constexpr int kLdsSumsMaxK = 64;                           // LDS partial sums up to k = 64
constexpr int kSortChunk = 1024;

struct KmWork {
  float* cent;     // [BH, k, 128]
  float* cc;       // [BH, k]
  long long* sums; // [BH, k, 128]
  unsigned* counts;// [BH, k]
  int32_t* labels; // [BH, N]
  int32_t* prev;   // [BH, N] labels as of the last accumulation
  int32_t* hist;   // [BH, nchunks, k]
};

// |c|^2 as a fmaf chain in channel order (one lane, reads the centroid from LDS).
__device__ float centroid_norm(const float* c) {
  float acc = 0.0f;
  for (int i = 0; i < kD; ++i) acc = __builtin_fmaf(c[i], c[i], acc);
  return acc;
}

// Two int8 digits of a value x of a row with max |row| = m: with inv = fl(32512 / m),
// X = RNE(x * inv) satisfies |X| <= 32512 and |x - X / inv| <= 1 / (2 inv).  One
// fused multiply-add t = fl(x * inv + (1.5 * 2^23 + 128)) rounds x * inv to X
// and leaves X + 128 in the low 16 bits of t (two's complement; t stays in
// [2^23, 2^24), where the float spacing is 1): byte 1 of t is the signed high
// digit h, byte 0 is l + 128, and X = 256 h + l with h in [-127, 127], l in
// [-128, 127].
constexpr float kDigitMagic = 12583040.0f;   // 1.5 * 2^23 + 128
__device__ __forceinline__ uint32_t digit_word(float x, float inv) {
  return __float_as_uint(__builtin_fmaf(x, inv, kDigitMagic));
}
// high digits (byte 1) and low digits (byte 0 ^ 0x80) of four digit words
__device__ __forceinline__ void digit_bytes(uint32_t t0, uint32_t t1, uint32_t t2, uint32_t t3, uint32_t& hi,
                                            uint32_t& lo) {
  const uint32_t a = __builtin_amdgcn_perm(t1, t0, 0x05010400u);   // t0.b0 t1.b0 t0.b1 t1.b1
  const uint32_t b = __builtin_amdgcn_perm(t3, t2, 0x05010400u);   // t2.b0 t3.b0 t2.b1 t3.b1
  hi = __builtin_amdgcn_perm(b, a, 0x07060302u);                   // t0.b1 t1.b1 t2.b1 t3.b1
  lo = __builtin_amdgcn_perm(b, a, 0x05040100u) ^ 0x80808080u;     // t0.b0 t1.b0 t2.b0 t3.b0
}

// value of lane l ^ 32 (V_PERMLANE32_SWAP, no LDS permute): with both operands
// x, each lane gets its own value in one result and that of lane l ^ 32 in the
// other, so the one that differs from x is the other half's (if neither
// differs, the two values are equal)
__device__ __forceinline__ int swap_halves(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return (int)(r[0] != (unsigned)x ? r[0] : r[1]);
}
__device__ __forceinline__ float swap_halves(float x) {
  return __int_as_float(swap_halves(__float_as_int(x)));
}

__global__ void __launch_bounds__(kD) kmeans_init(const uint16_t* __restrict__ V, int N, int k,
                                                  KmWork w) {
  const int c = blockIdx.x, bh = blockIdx.y, i = threadIdx.x;
  __shared__ float row[kD];
  const long long src = ((long long)c * N) / k;
  const float v = bf16_bits_to_f32(V[((long long)bh * N + src) * kD + i]);
  row[i] = v;
  const long long ci = ((long long)bh * k + c) * kD + i;
  w.cent[ci] = v;
  w.sums[ci] = 0;
  __syncthreads();
  if (i == 0) {
    w.cc[(long long)bh * k + c] = centroid_norm(row);
    w.counts[(long long)bh * k + c] = 0u;
  }
}

__global__ void __launch_bounds__(kAssignThreads) kmeans_assign(const uint16_t* __restrict__ V, int N, int k,
                                                                 KmWork w) {
  __shared__ unsigned cnt[256];
  const int bh = blockIdx.y, tid = threadIdx.x;
  // Centroids and |c|^2 are read with wave-uniform addresses: the compiler turns
  // them into scalar loads, so every FMA takes its centroid value from an SGPR
  // and the centroids cost no LDS bandwidth.
  const float* __restrict__ C = w.cent + (long long)bh * k * kD;
  const float* __restrict__ ccg = w.cc + (long long)bh * k;
  for (int c = tid; c < k; c += kAssignThreads) cnt[c] = 0u;
  __syncthreads();

  const long long base = (long long)blockIdx.x * kTokPerWG;
#pragma unroll 1
  for (int s = 0; s < kTokPerThread; ++s) {
    const long long j = base + tid + (long long)s * kAssignThreads;
    if (j >= N) break;
    const uint16_t* vp = V + ((long long)bh * N + j) * kD;
    float x[kD];
#pragma unroll
    for (int q = 0; q < kD / 8; ++q) {
      const uint4 raw = *reinterpret_cast<const uint4*>(vp + q * 8);
      const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[q * 8 + 2 * e] = __uint_as_float(wds[e] << 16);
        x[q * 8 + 2 * e + 1] = __uint_as_float(wds[e] & 0xFFFF0000u);
      }
    }
    int best = 0;
    float best_s = __builtin_inff();
    const int k4 = k & ~3;
#pragma unroll 1
    for (int c = 0; c < k4; c += 4) {
      float d0 = 0.0f, d1 = 0.0f, d2 = 0.0f, d3 = 0.0f;
#pragma unroll
      for (int i = 0; i < kD; ++i) {   // fixed order: channel 0..127
        d0 = __builtin_fmaf(x[i], C[(c + 0) * kD + i], d0);
        d1 = __builtin_fmaf(x[i], C[(c + 1) * kD + i], d1);
        d2 = __builtin_fmaf(x[i], C[(c + 2) * kD + i], d2);
        d3 = __builtin_fmaf(x[i], C[(c + 3) * kD + i], d3);
      }
      const float sc0 = __builtin_fmaf(-2.0f, d0, ccg[c + 0]);
      const float sc1 = __builtin_fmaf(-2.0f, d1, ccg[c + 1]);
      const float sc2 = __builtin_fmaf(-2.0f, d2, ccg[c + 2]);
      const float sc3 = __builtin_fmaf(-2.0f, d3, ccg[c + 3]);
      // strict comparisons in index order: the lowest index wins ties
      if (sc0 < best_s) { best_s = sc0; best = c + 0; }
      if (sc1 < best_s) { best_s = sc1; best = c + 1; }
      if (sc2 < best_s) { best_s = sc2; best = c + 2; }
      if (sc3 < best_s) { best_s = sc3; best = c + 3; }
    }
#pragma unroll 1
    for (int c = k4; c < k; ++c) {
      float d0 = 0.0f;
#pragma unroll
      for (int i = 0; i < kD; ++i) d0 = __builtin_fmaf(x[i], C[c * kD + i], d0);
      const float sc0 = __builtin_fmaf(-2.0f, d0, ccg[c]);
      if (sc0 < best_s) { best_s = sc0; best = c; }
    }
    w.labels[(long long)bh * N + j] = best;
    atomicAdd(&cnt[best], 1u);
  }
  __syncthreads();
  for (int c = tid; c < k; c += kAssignThreads)
    if (cnt[c]) atomicAdd(&w.counts[(long long)bh * k + c], cnt[c]);
}

// Screened assignment (k <= 64).  The distance of the fixed-order fp32 rule is
// the arbiter; a screen finds every token whose argmin it decides.
//  * The token's bf16 values and every centroid are coded as two int8 digits
//    per value with one factor per row (digit_word): x = (256 h + l) r + d with
//    r = 1 / fl(32512 / max|row|) and |d| <= r / 2.  V_MFMA_I32_32X32X32_I8 gives
//    the exact integer dot products D_hh of the high digits and D_x = D_hl + D_lh
//    of the mixed ones; the low-low term (|D_ll| <= 2^21) is dropped.
//  * The screened score s_a = cc - 512 r_v r_c (256 D_hh + D_x) differs from the
//    fixed-order score s_o by at most
//    B = 1.002 [ r_c |v|_1 + r_v |c|_1               (digit errors, times 2)
//              + (2^22 + 64) r_v r_c                 (dropped low-low term and the digit cross term)
//              + (2^-15 + 2^-17) |v|_1 max|c| ]      (fp32 chain of s_o; rounding of s_a)
//        + 2^-19 |cc|                               (rounding of s_a and of the comparison)
//    where the factor 1.002 covers the evaluation of B.  Per centroid, B =
//    A_c |v|_1 + r_v B_c + C_c with A_c, B_c, C_c from an LDS table.
//  * With U = min_c (s_a + B), only centroids with s_a - B <= U can be the
//    argmin.  A token with one such centroid takes it (all others score
//    strictly more); any other token is recomputed with the fixed-order
//    chain itself: lane c takes centroid c, the lowest index wins ties.  So is
//    every token, and every centroid counts as a candidate, whose max |x| lies
//    outside [2^-40, 2^40] (0 aside), where the rounding terms would not hold.
// Lane layout: lanes l and l + 32 share token l % 32 (channel halves of each
// 32-channel slice: the B operand of the MFMA); the output rows (centroids)
// 8(r/4) + 4(l/32) + r%4 of each 32-centroid block stay in lane l.
template <int kNB>   // 32-centroid blocks: (k + 31) / 32
__global__ void __launch_bounds__(kAssignThreads) kmeans_assign_mfma(const uint16_t* __restrict__ V, int N, int k,
                                                                      KmWork w) {
  __shared__ float Ct[kD][kLdsSumsMaxK + 1];   // centroids transposed (zero past k), padded against bank conflicts
  // centroid digits as MFMA A operands: [digit][slice][half][centroid][16 bytes]
  __shared__ __align__(16) uint4 cqs[2][4][2][kLdsSumsMaxK];
  __shared__ float ccs[kLdsSumsMaxK];      // |c|^2, +inf past k
  __shared__ float part[2][4][kLdsSumsMaxK];
  __shared__ float invs[kLdsSumsMaxK];     // fl(32512 / max|c|), 0 for a zero centroid
  __shared__ float4 tabA[kLdsSumsMaxK];    // {-512 r_c, A_c, B_c, cc} (zero and +inf past k)
  __shared__ float tabC[kLdsSumsMaxK];     // C_c
  __shared__ unsigned cnt[kLdsSumsMaxK];
  const int bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, g = lane >> 5, col = lane & 31;
  const float* __restrict__ C = w.cent + (long long)bh * k * kD;
  for (int idx = tid; idx < kLdsSumsMaxK * kD; idx += kAssignThreads) {
    const int c = idx / kD, i = idx % kD;
    Ct[i][c] = c < k ? C[idx] : 0.0f;
  }
  if (tid < kLdsSumsMaxK) {
    ccs[tid] = tid < k ? w.cc[(long long)bh * k + tid] : __builtin_inff();
    cnt[tid] = 0u;
  }
  __syncthreads();
  {  // per-centroid |c|_1 and max|c| over channel quarters
    const int c = tid & 63, q = tid >> 6;
    float l1 = 0.0f, mx = 0.0f;
    for (int i = 32 * q; i < 32 * q + 32; ++i) {
      l1 += fabsf(Ct[i][c]);
      mx = fmaxf(mx, fabsf(Ct[i][c]));
    }
    part[0][q][c] = l1;
    part[1][q][c] = mx;
  }
  __syncthreads();
  if (tid < kLdsSumsMaxK) {
    const int c = tid;
    const float l1 = (((part[0][0][c] + part[0][1][c]) + part[0][2][c]) + part[0][3][c]) * (1.0f + 0x1p-15f);
    const float mx = fmaxf(fmaxf(part[1][0][c], part[1][1][c]), fmaxf(part[1][2][c], part[1][3][c]));
    const float inv_c = mx > 0.0f ? 32512.0f / mx : 0.0f;
    const float rc = mx > 0.0f ? 1.0f / inv_c : 0.0f;
    // a centroid outside the screened range is a candidate for every token
    const bool ok = mx == 0.0f || (mx >= 0x1p-40f && mx <= 0x1p40f);
    invs[c] = inv_c;
    if (c < k) {
      tabA[c] = make_float4(-512.0f * rc, 1.002f * (rc + (0x1p-15f + 0x1p-17f) * mx),
                            1.002f * (l1 + 4194368.0f * rc), ccs[c]);   // 2^22 + 64
      tabC[c] = ok ? 0x1p-19f * fabsf(ccs[c]) : __builtin_inff();
    } else {
      tabA[c] = make_float4(0.0f, 0.0f, 0.0f, __builtin_inff());
      tabC[c] = 0.0f;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < 4 * 2 * kLdsSumsMaxK; idx += kAssignThreads) {
    const int c = idx % kLdsSumsMaxK, gg = (idx / kLdsSumsMaxK) % 2, s4 = idx / (2 * kLdsSumsMaxK);
    const float inv_c = invs[c];
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* col = &Ct[32 * s4 + 16 * gg + 4 * q][c];
      digit_bytes(digit_word(col[0], inv_c), digit_word(col[kLdsSumsMaxK + 1], inv_c),
                  digit_word(col[2 * (kLdsSumsMaxK + 1)], inv_c), digit_word(col[3 * (kLdsSumsMaxK + 1)], inv_c),
                  hw[q], lw[q]);
    }
    cqs[0][s4][gg][c] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    cqs[1][s4][gg][c] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
  __syncthreads();

  const int wave = tid >> 6;
  const long long wbase = (long long)blockIdx.x * kMTokWG + (long long)wave * (kMTokWG / 4);
  uint32_t raw[4][8];
  auto load_group = [&](long long t0) {
    const long long t = t0 + col;
    const uint16_t* vp = V + ((long long)bh * N + (t < N ? t : t0)) * kD;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 u = *reinterpret_cast<const uint4*>(vp + 32 * s4 + 16 * g + 8 * h);
        raw[s4][4 * h + 0] = u.x; raw[s4][4 * h + 1] = u.y; raw[s4][4 * h + 2] = u.z; raw[s4][4 * h + 3] = u.w;
      }
  };
  if (wbase < N) load_group(wbase);
#pragma unroll 1
  for (int grp = 0; grp < kMTokWG / 4 / 32; ++grp) {
    const long long t0 = wbase + 32 * grp;
    if (t0 >= N) break;
    const long long t = t0 + col;
    const bool live = t < N;
    // max |v| from the magnitude bits (they order like the values, two at a time
    // with V_PK_MAX_U16) and an upper bound of |v|_1 (V_DOT2_F32_BF16 against ones;
    // its rounding and any flush of subnormals stay far inside the 2^-15 margin)
    u16x2 mb = {0, 0};
    float l1 = 0.0f;
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t mag = raw[s4][q] & 0x7FFF7FFFu;
        mb = __builtin_elementwise_max(mb, __builtin_bit_cast(u16x2, mag));
        l1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, mag), ones, l1, false);
      }
    const uint32_t mbw = __builtin_bit_cast(uint32_t, mb);
    const float vmax_l = fmaxf(__uint_as_float(mbw << 16), __uint_as_float(mbw & 0xFFFF0000u));
    const float vmax = fmaxf(vmax_l, swap_halves(vmax_l));
    l1 = (l1 + swap_halves(l1)) * (1.0f + 0x1p-15f);
    const bool screenable = vmax == 0.0f || (vmax >= 0x1p-40f && vmax <= 0x1p40f);
    // inv need not be the correctly rounded quotient: any inv with vmax * inv
    // below 32639.5 keeps both digits in range, and r_v below is 1 / inv itself
    // (V_RCP_F32, within the 1.002 margin of the bound)
    const float inv = vmax > 0.0f ? 32512.0f * __builtin_amdgcn_rcpf(vmax) : 0.0f;
    const float sv = vmax > 0.0f ? __builtin_amdgcn_rcpf(inv) : 0.0f;   // r_v
    // token digits (digit_word): one fused multiply-add per value, the bytes
    // gathered four values at a time
    v4i bop[2][4];   // [high/low][slice]
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        uint32_t tw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ee = 4 * q4 + e;
          const uint32_t wd = raw[s4][ee >> 1];
          tw[e] = digit_word(__uint_as_float((ee & 1) ? (wd & 0xFFFF0000u) : (wd << 16)), inv);
        }
        uint32_t wh, wl;
        digit_bytes(tw[0], tw[1], tw[2], tw[3], wh, wl);
        bop[0][s4][q4] = (int)wh;
        bop[1][s4][q4] = (int)wl;
      }
    // prefetch of the next group, unconditional (the last group reloads itself)
    // so that the compiler keeps one copy of the row registers
    load_group(grp + 1 < kMTokWG / 4 / 32 && t0 + 32 < N ? t0 + 32 : t0);
    // screened scores s_a = cc - 512 r_v r_c D (D = 256 D_hh + D_x) of
    // centroids 32b + 8(r/4) + 4g + r%4 (this lane's rows) with their bounds:
    // keep s_a - B, and U = min (s_a + B) over the token's centroids
    float lo[2][16];
    float U = __builtin_inff();
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (b < kNB) {
        v16i acc, accx;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = accx[r] = 0;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const uint4 ah = cqs[0][s4][g][32 * b + col], al = cqs[1][s4][g][32 * b + col];
          const v4i aoh = {(int)ah.x, (int)ah.y, (int)ah.z, (int)ah.w};
          const v4i aol = {(int)al.x, (int)al.y, (int)al.z, (int)al.w};
          acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(aoh, bop[0][s4], acc, 0, 0, 0);
          accx = __builtin_amdgcn_mfma_i32_32x32x32_i8(aol, bop[0][s4], accx, 0, 0, 0);
          accx = __builtin_amdgcn_mfma_i32_32x32x32_i8(aoh, bop[1][s4], accx, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 32 * b + 8 * (r >> 2) + 4 * g + (r & 3);
          const float4 ta = tabA[c];
          // |256 D_hh + D_x| < 2^30 (|D_hh| < 2^21, |D_x| < 2^22): exact in int32
          const int di = acc[r] * 256 + accx[r];
          const float sa = __builtin_fmaf((float)di, sv * ta.x, ta.w);
          const float bd = __builtin_fmaf(ta.y, l1, __builtin_fmaf(ta.z, sv, tabC[c]));
          lo[b][r] = sa - bd;
          U = fminf(U, sa + bd);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) lo[b][r] = __builtin_inff();
      }
    }
    U = fminf(U, swap_halves(U));
    // candidates: centroids that can still be the argmin (cand holds the row
    // index without this lane's 4g)
    int ncand = 0, cand = -1;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool in = lo[b][r] <= U;
        ncand += in ? 1 : 0;
        cand = in ? 32 * b + 8 * (r >> 2) + (r & 3) : cand;
      }
    cand = cand < 0 ? -1 : cand + 4 * g;
    ncand += swap_halves(ncand);
    cand = max(cand, swap_halves(cand));
    int label = cand;
    // fixed-order recheck of the tokens the screen leaves open
    unsigned long long open = __ballot(live && (ncand != 1 || !screenable) && g == 0);
    while (open) {
      const int tl = __builtin_ctzll(open);
      open &= open - 1;
      // the token's row in one coalesced load (lane l: channels 2l, 2l + 1); the
      // chain takes each value from its lane with V_READLANE (a scalar operand)
      const uint32_t wrow = reinterpret_cast<const uint32_t*>(V + ((long long)bh * N + t0 + tl) * kD)[lane];
      float d = 0.0f;
      const int c = lane;   // Ct is zero past k
#pragma unroll 16
      for (int i2 = 0; i2 < kD / 2; ++i2) {   // fixed order: channel 0..127
        const uint32_t wv = __builtin_amdgcn_readlane(wrow, i2);
        d = __builtin_fmaf(__uint_as_float(wv << 16), Ct[2 * i2][c], d);
        d = __builtin_fmaf(__uint_as_float(wv & 0xFFFF0000u), Ct[2 * i2 + 1][c], d);
      }
      float sc = c < k ? __builtin_fmaf(-2.0f, d, ccs[c]) : __builtin_inff();
      int bi = c;
      // argmin over the lanes, lowest index on ties
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float so = __shfl_xor(sc, o);
        const int io = __shfl_xor(bi, o);
        if (so < sc || (so == sc && io < bi)) {
          sc = so;
          bi = io;
        }
      }
      if (col == tl) label = min(max(bi, 0), k - 1);   // in range even for non-finite data
    }
    if (live && g == 0) {
      label = min(max(label, 0), k - 1);   // a lone candidate is always a real centroid; kept as a guard
      w.labels[(long long)bh * N + t] = label;
      atomicAdd(&cnt[label], 1u);
    }
  }
  __syncthreads();
  for (int c = tid; c < k; c += kAssignThreads)
    if (cnt[c]) atomicAdd(&w.counts[(long long)bh * k + c], cnt[c]);
}

// Fixed-point sums of every cluster: int64 sum of rint(v * 2^24) per (cluster,
// channel).  Tokens go one at a time with lanes over channels: lane l takes
// channels 2l and 2l+1 (one 32-bit load), and the LDS partials are laid out so
// that both adds of a token hit 64 consecutive 8-byte slots of the token's
// cluster row (slot h*64 + l holds channel 2l + h); they never collide.  The
// integer adds are order-free, so any split of the tokens gives the same sums.
// The sums persist across iterations: the first pass (kmeans_accum) adds every
// token; each later pass (kmeans_accum_moved) adds only the tokens whose label
// moved since the last pass to their new cluster and subtracts them from their
// old one, which leaves the same integers as a full recount.  Both passes end
// by recording the labels they accounted for.

// rint(v * 2^24) of the two channels of a row word, added to (sign +1) or
// subtracted from (sign -1) cluster c's partials.  The int32 conversion is exact
// when |v| < 128 (largest bf16 below 128: 127.5 * 2^24 < 2^31); the float ->
// int64 sequence gives the same integers for any finite v.
template <bool kLdsSums, bool kSmall>
__device__ __forceinline__ void add_row_word(uint32_t word, int c, bool negate, int ln,
                                             unsigned long long* psum, unsigned long long* gs) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float xv = __uint_as_float(h ? (word & 0xFFFF0000u) : (word << 16));
    const float r = __builtin_rintf(xv * 16777216.0f);
    long long qv = kSmall ? (long long)(int)r : (long long)r;
    if (negate) qv = -qv;
    if (kLdsSums) atomicAdd(&psum[c * kD + 64 * h + ln], (unsigned long long)qv);
    else atomicAdd(&gs[(long long)c * kD + 2 * ln + h], (unsigned long long)qv);
  }
}

// |v| < 128 (and finite) for both channels of every word, over the wavefront
template <int kN>
__device__ __forceinline__ bool words_small(const uint32_t (&raw)[kN]) {
  u16x2 mb = {0, 0};
#pragma unroll
  for (int b = 0; b < kN; ++b) mb = __builtin_elementwise_max(mb, __builtin_bit_cast(u16x2, raw[b] & 0x7FFF7FFFu));
  return __all(mb[0] < 0x4300u && mb[1] < 0x4300u);
}

template <bool kLdsSums>
__device__ __forceinline__ void flush_partials(int k, int tid, const unsigned long long* psum,
                                               unsigned long long* gs) {
  if (kLdsSums) {
    __syncthreads();
    for (int idx = tid; idx < k * kD; idx += kAccThreads) {
      const unsigned long long v = psum[idx];
      const int c = idx / kD, slot = idx % kD;
      if (v) atomicAdd(&gs[(long long)c * kD + 2 * (slot & 63) + (slot >> 6)], v);
    }
  }
}

template <bool kLdsSums>
__global__ void __launch_bounds__(kAccThreads) kmeans_accum(const uint16_t* __restrict__ V, int N, int k,
                                                              KmWork w) {
  extern __shared__ __align__(16) unsigned long long psum[];   // [k][128] when kLdsSums
  // the wavefront index made uniform for the compiler: token indices, labels and
  // the beyond-N test then live in scalar registers
  const int bh = blockIdx.y, tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), ln = tid & 63;
  if (kLdsSums)
    for (int idx = tid; idx < k * kD; idx += kAccThreads) psum[idx] = 0ull;
  __syncthreads();
  unsigned long long* gs = reinterpret_cast<unsigned long long*>(w.sums) + (long long)bh * k * kD;
  const int32_t* __restrict__ lab = w.labels + (long long)bh * N;
  const uint32_t* __restrict__ V32 = reinterpret_cast<const uint32_t*>(V + (long long)bh * N * kD);
  constexpr int kPerWave = kAccTok / (kAccThreads / 64);
  constexpr int kBatch = 32;
  const long long j_begin = (long long)blockIdx.x * kAccTok + (long long)wv * kPerWave;
#pragma unroll 1
  for (int j0 = 0; j0 < kPerWave; j0 += kBatch) {
    if (j_begin + j0 >= N) break;
    uint32_t raw[kBatch];
    int cl[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const long long j = j_begin + j0 + b;
      const long long jj = j < N ? j : (long long)N - 1;
      cl[b] = j < N ? lab[jj] : -1;   // uniform address: a scalar load
      raw[b] = V32[jj * (kD / 2) + ln];
    }
    auto add_batch = [&](auto small_tag) {
#pragma unroll
      for (int b = 0; b < kBatch; ++b)
        if (cl[b] >= 0)   // not beyond N (uniform across the wavefront)
          add_row_word<kLdsSums, decltype(small_tag)::value>(raw[b], cl[b], false, ln, psum, gs);
    };
    if (words_small(raw)) add_batch(std::true_type{});
    else add_batch(std::false_type{});
  }
  int32_t* __restrict__ prv = w.prev + (long long)bh * N;
  for (int q = ln; q < kPerWave; q += 64) {
    const long long j = j_begin + q;
    if (j < N) prv[j] = lab[j];
  }
  flush_partials<kLdsSums>(k, tid, psum, gs);
}

// The later passes: each wavefront compares the labels of its 256 tokens with
// the recorded ones (coalesced loads, one ballot per 64 tokens) and reads the
// rows of the moved tokens only, eight at a time.
template <bool kLdsSums>
__global__ void __launch_bounds__(kAccThreads) kmeans_accum_moved(const uint16_t* __restrict__ V, int N, int k,
                                                                    KmWork w) {
  extern __shared__ __align__(16) unsigned long long psum[];   // [k][128] when kLdsSums
  const int bh = blockIdx.y, tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), ln = tid & 63;
  if (kLdsSums)
    for (int idx = tid; idx < k * kD; idx += kAccThreads) psum[idx] = 0ull;
  __syncthreads();
  unsigned long long* gs = reinterpret_cast<unsigned long long*>(w.sums) + (long long)bh * k * kD;
  const int32_t* __restrict__ lab = w.labels + (long long)bh * N;
  int32_t* __restrict__ prv = w.prev + (long long)bh * N;
  const uint32_t* __restrict__ V32 = reinterpret_cast<const uint32_t*>(V + (long long)bh * N * kD);
  constexpr int kPerWave = kAccTok / (kAccThreads / 64);
  const long long j_begin = (long long)blockIdx.x * kAccTok + (long long)wv * kPerWave;
  int nl[kPerWave / 64], ol[kPerWave / 64];
#pragma unroll
  for (int q = 0; q < kPerWave / 64; ++q) {
    const long long j = j_begin + 64 * q + ln;
    nl[q] = j < N ? lab[j] : 0;
    ol[q] = j < N ? prv[j] : 0;
  }
#pragma unroll
  for (int q = 0; q < kPerWave / 64; ++q) {
    unsigned long long m = __ballot(nl[q] != ol[q]);
    while (m) {   // uniform
      uint32_t raw[8];
      int cn[8], co[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        cn[u] = -1;
        co[u] = -1;
        raw[u] = 0u;
        if (m) {
          const int tl = __builtin_ctzll(m);
          m &= m - 1;
          cn[u] = __builtin_amdgcn_readlane(nl[q], tl);
          co[u] = __builtin_amdgcn_readlane(ol[q], tl);
          raw[u] = V32[(j_begin + 64 * q + tl) * (kD / 2) + ln];
        }
      }
      auto add_moved = [&](auto small_tag) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (cn[u] >= 0) {   // uniform
            add_row_word<kLdsSums, decltype(small_tag)::value>(raw[u], cn[u], false, ln, psum, gs);
            add_row_word<kLdsSums, decltype(small_tag)::value>(raw[u], co[u], true, ln, psum, gs);
          }
      };
      if (words_small(raw)) add_moved(std::true_type{});
      else add_moved(std::false_type{});
    }
    const long long j = j_begin + 64 * q + ln;
    if (j < N && nl[q] != ol[q]) prv[j] = nl[q];
  }
  flush_partials<kLdsSums>(k, tid, psum, gs);
}

__global__ void __launch_bounds__(kD) kmeans_update(int k, KmWork w) {
  const int c = blockIdx.x, bh = blockIdx.y, i = threadIdx.x;
  __shared__ float row[kD];
  const long long ci = ((long long)bh * k + c) * kD + i;
  const unsigned n = w.counts[(long long)bh * k + c];
  float v = w.cent[ci];
  if (n > 0) {
    const double s = (double)w.sums[ci];
    v = (float)((s * 0x1p-24) / (double)n);
    w.cent[ci] = v;
  }
  row[i] = v;
  __syncthreads();
  if (i == 0) {
    w.cc[(long long)bh * k + c] = centroid_norm(row);
    w.counts[(long long)bh * k + c] = 0u;
  }
}

__global__ void __launch_bounds__(256) sort_hist(int N, int k, int nchunks, KmWork w) {
  extern __shared__ unsigned hs[];
  const int chunk = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  for (int c = tid; c < k; c += 256) hs[c] = 0u;
  __syncthreads();
  const long long base = (long long)chunk * kSortChunk;
  for (int s = 0; s < kSortChunk / 256; ++s) {
    const long long j = base + tid + s * 256;
    if (j < N) atomicAdd(&hs[w.labels[(long long)bh * N + j]], 1u);
  }
  __syncthreads();
  for (int c = tid; c < k; c += 256) w.hist[((long long)bh * nchunks + chunk) * k + c] = (int32_t)hs[c];
}

// Turns the per-chunk histograms into the first output slot of every (chunk, label).
__global__ void __launch_bounds__(256) sort_scan(int k, int nchunks, KmWork w) {
  __shared__ int tot[256];
  const int bh = blockIdx.x, c = threadIdx.x;
  int32_t* hist = w.hist + (long long)bh * nchunks * k;
  int t = 0;
  if (c < k)
    for (int ch = 0; ch < nchunks; ++ch) t += hist[(long long)ch * k + c];
  tot[c] = c < k ? t : 0;
  __syncthreads();
  if (c == 0) {
    int run = 0;
    for (int q = 0; q < k; ++q) {
      const int n = tot[q];
      tot[q] = run;
      run += n;
    }
  }
  __syncthreads();
  if (c < k) {
    int run = tot[c];
    for (int ch = 0; ch < nchunks; ++ch) {
      const int n = hist[(long long)ch * k + c];
      hist[(long long)ch * k + c] = run;
      run += n;
    }
  }
}

// Stable scatter of one 1024-token chunk: wavefront w takes tokens 256w ..
// 256w + 255 in steps of 64.  In a step, the lanes with the same label are
// found by matching the label bits with ballots; a lane's rank is the count of
// its label so far in the wavefront plus the matching lanes below it.  Ranks of
// later wavefronts are offset by the counts of the earlier ones, so positions
// follow the original token order within every label.
__global__ void __launch_bounds__(256) sort_scatter(int N, int k, int nchunks, KmWork w,
                                                    int32_t* __restrict__ perm) {
  static_assert(kSortChunk == 4 * 256, "four wavefronts of 256 tokens");
  __shared__ int wcnt[4][256];   // per-wavefront label counts (k <= 256)
  const int chunk = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const long long base = (long long)chunk * kSortChunk;
  const int len = (int)min((long long)kSortChunk, (long long)N - base);
  for (int q = tid; q < 4 * 256; q += 256) (&wcnt[0][0])[q] = 0;
  __syncthreads();
  const int nbits = k <= 1 ? 0 : 32 - __clz(k - 1);
  const unsigned long long below = (1ull << lane) - 1ull;
  int lbl[4], rank[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int j = wave * 256 + s * 64 + lane;
    const bool valid = j < len;
    const int label = valid ? w.labels[(long long)bh * N + base + j] : 0;
    unsigned long long match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (label >> b) & 1;
      const unsigned long long bal = __ballot(bit);
      match &= bit ? bal : ~bal;
    }
    lbl[s] = label;
    rank[s] = valid ? wcnt[wave][label] + __popcll(match & below) : 0;
    // the highest lane of each label group adds the group's size
    if (valid && (match >> lane) == 1ull) wcnt[wave][label] += __popcll(match);
  }
  __syncthreads();
  const int32_t* off = w.hist + ((long long)bh * nchunks + chunk) * k;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int j = wave * 256 + s * 64 + lane;
    if (j < len) {
      int pre = 0;
      for (int ww = 0; ww < wave; ++ww) pre += wcnt[ww][lbl[s]];
      perm[(long long)bh * N + off[lbl[s]] + pre + rank[s]] = (int32_t)(base + j);
    }
  }
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct KmLayout {
  size_t cent, cc, sums, counts, labels, prev, hist, total;
};

static KmLayout km_layout(long long BH, long long N, int k) {
  KmLayout L;
  const long long nchunks = (N + kSortChunk - 1) / kSortChunk;
  size_t o = 0;
  L.cent = o;   o += align256(sizeof(float) * BH * k * kD);
  L.cc = o;     o += align256(sizeof(float) * BH * k);
  L.sums = o;   o += align256(sizeof(long long) * BH * k * kD);
  L.counts = o; o += align256(sizeof(unsigned) * BH * k);
  L.labels = o; o += align256(sizeof(int32_t) * BH * N);
  L.prev = o;   o += align256(sizeof(int32_t) * BH * N);
  L.hist = o;   o += align256(sizeof(int32_t) * BH * nchunks * k);
  L.total = o;
  return L;
}

}  // namespace vc

using namespace vc;

extern "C" size_t vc_vsmooth_group_workspace(int B, int H, int N, int d, int k) {
  if (B < 1 || H < 1 || N < 1 || d != kD || k < 1 || k > 256) return 0;
  return km_layout((long long)B * H, N, k).total;
}

extern "C" int vc_vsmooth_group(const uint16_t* V, int B, int H, int N, int d, int k, int iters,
                                int32_t* perm, int32_t* labels, float* centroids, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (d != kD) return VC_ERR_UNSUPPORTED;
  if (!V || !perm || B < 1 || H < 1 || N < 1 || k < 1 || k > 256 || iters < 1) return VC_ERR_INVALID_ARG;
  if ((long long)B * H > 65535) return VC_ERR_INVALID_ARG;
  const long long BH = (long long)B * H;
  const KmLayout L = km_layout(BH, N, k);
  if (!workspace || workspace_bytes < L.total) return VC_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  KmWork w;
  w.cent = centroids ? centroids : reinterpret_cast<float*>(ws + L.cent);
  w.cc = reinterpret_cast<float*>(ws + L.cc);
  w.sums = reinterpret_cast<long long*>(ws + L.sums);
  w.counts = reinterpret_cast<unsigned*>(ws + L.counts);
  w.labels = labels ? labels : reinterpret_cast<int32_t*>(ws + L.labels);
  w.prev = reinterpret_cast<int32_t*>(ws + L.prev);
  w.hist = reinterpret_cast<int32_t*>(ws + L.hist);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int nchunks = (N + kSortChunk - 1) / kSortChunk;
  const bool lds_sums = k <= kLdsSumsMaxK;
  const size_t lds = lds_sums ? sizeof(unsigned long long) * (size_t)k * kD : 0;
  const dim3 gA((N + kTokPerWG - 1) / kTokPerWG, (unsigned)BH);
  const dim3 gS((N + kAccTok - 1) / kAccTok, (unsigned)BH);
  // dynamic LDS above the default limit (cheap; set on every call, no state kept)
  if (lds_sums) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kmeans_accum<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kmeans_accum_moved<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  }
  hipLaunchKernelGGL(kmeans_init, dim3(k, (unsigned)BH), dim3(kD), 0, st, V, N, k, w);
  const dim3 gM((N + kMTokWG - 1) / kMTokWG, (unsigned)BH);
  for (int it = 0; it < iters; ++it) {
    if (k <= kLdsSumsMaxK) {   // screened int8 MFMA pass with a fixed-order recheck
      if (k > 32)
        hipLaunchKernelGGL(kmeans_assign_mfma<2>, gM, dim3(kAssignThreads), 0, st, V, N, k, w);
      else
        hipLaunchKernelGGL(kmeans_assign_mfma<1>, gM, dim3(kAssignThreads), 0, st, V, N, k, w);
    } else
      hipLaunchKernelGGL(kmeans_assign, gA, dim3(kAssignThreads), 0, st, V, N, k, w);
    // the labels of the last assignment give the permutation; the update after
    // it only matters when the caller asks for the centroids
    if (it + 1 == iters && !centroids) break;
    // the first pass counts every token, later passes only the moved ones
    if (lds_sums && it == 0)
      hipLaunchKernelGGL(kmeans_accum<true>, gS, dim3(kAccThreads), lds, st, V, N, k, w);
    else if (lds_sums)
      hipLaunchKernelGGL(kmeans_accum_moved<true>, gS, dim3(kAccThreads), lds, st, V, N, k, w);
    else if (it == 0)
      hipLaunchKernelGGL(kmeans_accum<false>, gS, dim3(kAccThreads), 0, st, V, N, k, w);
    else
      hipLaunchKernelGGL(kmeans_accum_moved<false>, gS, dim3(kAccThreads), 0, st, V, N, k, w);
    hipLaunchKernelGGL(kmeans_update, dim3(k, (unsigned)BH), dim3(kD), 0, st, k, w);
  }
  hipLaunchKernelGGL(sort_hist, dim3(nchunks, (unsigned)BH), dim3(256), sizeof(unsigned) * k, st, N, k,
                     nchunks, w);
  hipLaunchKernelGGL(sort_scan, dim3((unsigned)BH), dim3(256), 0, st, k, nchunks, w);
  hipLaunchKernelGGL(sort_scatter, dim3(nchunks, (unsigned)BH), dim3(256), 0, st, N, k, nchunks, w, perm);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return vc_set_hip_error((int)e);
  return VC_OK;
}
