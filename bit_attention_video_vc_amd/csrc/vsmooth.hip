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
//   kmeans_init     centroid c <- V[floor(c*N/k)], zero the accumulators, |c|^2
//   kmeans_assign   labels and counts: one token per lane, four independent FMA
//                   chains (centroids read through the scalar cache: uniform
//                   addresses)
//   kmeans_accum    fixed-point sums: tokens one at a time, lanes over channels,
//                   into LDS (k <= 64; conflict-free), then one global atomic
//                   per non-zero partial of the 2048-token block
//   kmeans_update   new centroids, zero the accumulators, |c|^2
//   sort_hist / sort_scan / sort_scatter   stable counting sort by label
#include "vc_common.h"

namespace vc {

constexpr int kAssignThreads = 256;
constexpr int kTokPerThread = 2;
constexpr int kTokPerWG = kAssignThreads * kTokPerThread;  // 512 tokens
constexpr int kAccThreads = 256;
constexpr int kAccTok = 2048;                              // tokens per accumulation workgroup
constexpr int kLdsSumsMaxK = 64;                           // LDS partial sums up to k = 64
constexpr int kSortChunk = 1024;

struct KmWork {
  float* cent;     // [BH, k, 128]
  float* cc;       // [BH, k]
  long long* sums; // [BH, k, 128]
  unsigned* counts;// [BH, k]
  int32_t* labels; // [BH, N]
  int32_t* hist;   // [BH, nchunks, k]
};

// |c|^2 as a fmaf chain in channel order (one lane, reads the centroid from LDS).
__device__ float centroid_norm(const float* c) {
  float acc = 0.0f;
  for (int i = 0; i < kD; ++i) acc = __builtin_fmaf(c[i], c[i], acc);
  return acc;
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

// Fixed-point sums of every cluster: int64 sum of rint(v * 2^24) per (cluster,
// channel).  Tokens go one at a time with lanes over channels: lane l takes
// channels 2l and 2l+1 (one 32-bit load), and the LDS partials are laid out so
// that both adds of a token hit 64 consecutive 8-byte slots of the token's
// cluster row (slot h*64 + l holds channel 2l + h); they never collide.  The
// integer adds are order-free, so any split of the tokens gives the same sums.
template <bool kLdsSums>
__global__ void __launch_bounds__(kAccThreads) kmeans_accum(const uint16_t* __restrict__ V, int N, int k,
                                                              KmWork w) {
  extern __shared__ __align__(16) unsigned long long psum[];   // [k][128] when kLdsSums
  const int bh = blockIdx.y, tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
  if (kLdsSums)
    for (int idx = tid; idx < k * kD; idx += kAccThreads) psum[idx] = 0ull;
  __syncthreads();
  unsigned long long* gs = reinterpret_cast<unsigned long long*>(w.sums) + (long long)bh * k * kD;
  const int32_t* __restrict__ lab = w.labels + (long long)bh * N;
  const uint32_t* __restrict__ V32 = reinterpret_cast<const uint32_t*>(V + (long long)bh * N * kD);
  constexpr int kPerWave = kAccTok / (kAccThreads / 64);
  constexpr int kBatch = 16;
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
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (cl[b] < 0) continue;   // beyond N (uniform across the wavefront)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float xv = __uint_as_float(h ? (raw[b] & 0xFFFF0000u) : (raw[b] << 16));
        const long long qv = (long long)__builtin_rintf(xv * 16777216.0f);
        if (kLdsSums) atomicAdd(&psum[cl[b] * kD + 64 * h + ln], (unsigned long long)qv);
        else atomicAdd(&gs[(long long)cl[b] * kD + 2 * ln + h], (unsigned long long)qv);
      }
    }
  }
  if (kLdsSums) {
    __syncthreads();
    for (int idx = tid; idx < k * kD; idx += kAccThreads) {
      const unsigned long long v = psum[idx];
      const int c = idx / kD, slot = idx % kD;
      if (v) atomicAdd(&gs[(long long)c * kD + 2 * (slot & 63) + (slot >> 6)], v);
    }
  }
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
  w.sums[ci] = 0;
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

__global__ void __launch_bounds__(256) sort_scatter(int N, int k, int nchunks, KmWork w,
                                                    int32_t* __restrict__ perm) {
  __shared__ int lab[kSortChunk];
  const int chunk = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const long long base = (long long)chunk * kSortChunk;
  const int len = (int)min((long long)kSortChunk, (long long)N - base);
  for (int q = tid; q < kSortChunk; q += 256) lab[q] = q < len ? w.labels[(long long)bh * N + base + q] : -1;
  __syncthreads();
  int mine[kSortChunk / 256], rank[kSortChunk / 256];
#pragma unroll
  for (int s = 0; s < kSortChunk / 256; ++s) {
    mine[s] = lab[tid + s * 256];
    rank[s] = 0;
  }
  // rank = number of earlier tokens of the chunk with the same label (stable order)
  for (int q = 0; q < len; ++q) {
    const int lq = lab[q];
#pragma unroll
    for (int s = 0; s < kSortChunk / 256; ++s) rank[s] += (lq == mine[s] && q < tid + s * 256) ? 1 : 0;
  }
  const int32_t* off = w.hist + ((long long)bh * nchunks + chunk) * k;
#pragma unroll
  for (int s = 0; s < kSortChunk / 256; ++s) {
    const int j = tid + s * 256;
    if (j < len) perm[(long long)bh * N + off[mine[s]] + rank[s]] = (int32_t)(base + j);
  }
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct KmLayout {
  size_t cent, cc, sums, counts, labels, hist, total;
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
  w.hist = reinterpret_cast<int32_t*>(ws + L.hist);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int nchunks = (N + kSortChunk - 1) / kSortChunk;
  const bool lds_sums = k <= kLdsSumsMaxK;
  const size_t lds = lds_sums ? sizeof(unsigned long long) * (size_t)k * kD : 0;
  const dim3 gA((N + kTokPerWG - 1) / kTokPerWG, (unsigned)BH);
  const dim3 gS((N + kAccTok - 1) / kAccTok, (unsigned)BH);
  // dynamic LDS above the default limit (cheap; set on every call, no state kept)
  if (lds_sums)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kmeans_accum<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(kmeans_init, dim3(k, (unsigned)BH), dim3(kD), 0, st, V, N, k, w);
  for (int it = 0; it < iters; ++it) {
    hipLaunchKernelGGL(kmeans_assign, gA, dim3(kAssignThreads), 0, st, V, N, k, w);
    if (lds_sums)
      hipLaunchKernelGGL(kmeans_accum<true>, gS, dim3(kAccThreads), lds, st, V, N, k, w);
    else
      hipLaunchKernelGGL(kmeans_accum<false>, gS, dim3(kAccThreads), 0, st, V, N, k, w);
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
