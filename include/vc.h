/*
 * vc.h -- C ABI of the VC-Attention hot path for AMD Instinct MI355X (gfx950).
 *
 * The method (four web pages about "VC-Attention: Value Smoothing and Softmax
 * Casting for Low-bit Attention"):
 *   V-Smooth  -- per batch and head, cluster the Value tokens with k-means,
 *                reorder Key and Value jointly by cluster label, subtract each
 *                128-token block's mean from Value, quantise only the residual,
 *                and add the means back from the online-softmax row sums as one
 *                outer product per block (paper digest, V-Smooth paragraph;
 *                news article, section "V-Smooth", items Group/Demean/Restore).
 *   ExpCast-FP8 -- write each E4M3 probability byte straight from the
 *                log-domain score with one fused multiply-add, round to nearest
 *                even, clip to the normal range, beta = -0.35 (paper digest,
 *                ExpCast-FP8 paragraph; news article, section "ExpCast-FP8").
 * The pages publish no API; these calls follow their statement of the problem.
 *
 * Conventions for every call
 *   - Every pointer argument is DEVICE memory owned by the caller, except where
 *     a comment says otherwise.  Arrays are dense and row-major unless a layout
 *     is spelled out.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued on
 *     it asynchronously; no call allocates, frees or synchronises.
 *   - Errors in the arguments are reported synchronously as a negative
 *     vc_status and nothing is enqueued.  A failed kernel launch returns
 *     VC_ERR_HIP (vc_last_hip_error() gives the HIP code).  Faults during a
 *     kernel surface at the caller's next synchronisation.
 *   - Shapes: B batches, H heads, N tokens per (batch, head), d = 128 channels.
 *     nb = ceil(N / 128) blocks; Np = 128 * nb padded rows.  Rows >= N of every
 *     code array are written as zero bytes.
 *   - Preconditions not checked: inputs are finite and |V| < 2^14.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Calls may run concurrently on different streams when their output and
 *     workspace buffers do not overlap.  The only state the library keeps is the
 *     HIP error code of the calling thread's last failed launch
 *     (vc_last_hip_error), held per thread.
 */
#ifndef VC_ATTN_VC_H
#define VC_ATTN_VC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum vc_status {
  VC_OK = 0,
  VC_ERR_INVALID_ARG = -1, /* null required pointer, N < 1, B/H < 1, k out of [1,256], iters < 1, or N
                              past 16,777,215 where a head's bytes must fit a 32-bit buffer record count */
  VC_ERR_UNSUPPORTED = -2, /* d != 128, unknown p_mode / v_format, or a mode pairing not built */
  VC_ERR_WORKSPACE = -3,   /* workspace pointer null or smaller than the *_workspace() size */
  VC_ERR_HIP = -4,         /* a HIP launch failed; see vc_last_hip_error() */
  VC_ERR_SCRATCH = -5      /* problem too large for the fixed scratch of an allocation-free entry point */
};

/* How the P tile (softmax numerator) is produced inside the attention kernel. */
enum vc_p_mode {
  VC_P_EXPCAST = 0,      /* ExpCast-FP8: code = RNE(fmaf(S, 8*kap, 55.65 - 8*mx)), codes < 8 -> 0 */
  VC_P_FP32EXP_E4M3 = 1, /* conventional: p = exp2(S*kap - mx) in fp32, then E4M3 (RNE) */
  VC_P_FP32_BF16 = 2     /* fp32 softmax, P rounded to bf16 (the 4-bit path; no ExpCast there) */
};

/* Format of the V residual codes. */
enum vc_v_format {
  VC_V_E4M3 = 0,  /* per-(b,h,channel) scaled E4M3 (8-bit path) */
  VC_V_NVFP4 = 1, /* E2M1 values, E4M3 scale per 16 tokens, fp32 scale per (b,h) (4-bit path) */
  VC_V_MXFP4 = 2  /* E2M1 values, E8M0 scale per 32 tokens (MI355X block-scaled FP4 MFMA; 4-bit path) */
};

/* ------------------------------------------------------------------------
 * V-Smooth grouping: k-means over Value tokens per (batch, head), then a stable
 * sort by cluster label (paper digest, V-Smooth paragraph: k-means runs per batch
 * and head over the Value tokens at inference time, and Key and Value are
 * reordered together by label; news article, "V-Smooth", item Group).
 *
 * Arithmetic (fixed so that the result is reproducible bit for bit):
 *   init     centroid c = V[floor(c*N/k)] (as fp32)
 *   assign   dot = fmaf chain over channels 0..127 from 0, cc = same for c.c,
 *            score = fmaf(-2, dot, cc), label = argmin, lowest c on ties
 *   update   int64 sums of llrint(v*2^24) per (cluster, channel), counts;
 *            centroid = (float)((double)sum * 2^-24 / (double)count);
 *            an empty cluster keeps its centroid
 *   iters    (assign, update) repeated `iters` times; labels from the last assign
 *   sort     stable counting sort: clusters ascending, tokens of a cluster in
 *            original order
 *
 * V          bf16 [B,H,N,128]
 * perm       out int32 [B,H,N]: perm[b,h,j'] = source token of permuted slot j'
 * labels     out int32 [B,H,N] cluster label of each ORIGINAL token (nullable)
 * centroids  out fp32 [B,H,k,128] after the last update (nullable)
 * workspace  device scratch of at least vc_vsmooth_group_workspace() bytes
 * ------------------------------------------------------------------------ */
size_t vc_vsmooth_group_workspace(int B, int H, int N, int d, int k);
int vc_vsmooth_group(const uint16_t* V, int B, int H, int N, int d, int k, int iters,
                     int32_t* perm, int32_t* labels, float* centroids,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Fused gather + block mean + quantisation (paper digest, V-Smooth and
 * preprocessing paragraphs: 128-row blocks subtract their mean, the residual
 * is quantised -- per-channel E4M3 on the 8-bit path, NVFP4 on the 4-bit path --
 * the mean is a 16-bit vector; mean, gather and quantisation are fused and no
 * high-precision intermediate goes back to memory).
 *
 * Arithmetic:
 *   K, V are gathered by perm; blocks are 128 permuted rows (last may be partial).
 *   mean_t   = bf16_RNE( fp32 sum over ascending rows / n_t )
 *   R        = fp32(v) - fp32(mean_t)
 *   E4M3 V   amax_c over all N rows of |R|; sv_c = amax_c/448 (0 if amax_c = 0);
 *            code = E4M3_RNE_SAT( R * (448/amax_c) )
 *   NVFP4 V  St = amax_all/2688 per (b,h); per channel and 16 consecutive
 *            permuted rows (inside a block): sg = E4M3( g_amax / (6*St) ),
 *            nibble = E2M1_RNE_SAT( R / (dec(sg)*St) )
 *   MXFP4 V  per channel, groups of 32 permuted rows of a block: rows 64h+16g+[0,16)
 *            and 64h+32+16g+[0,16) (h, g in {0,1}); X = 2^(floor(log2 g_amax) - 2),
 *            E8M0 code clamped to [0,254] (0 for an all-zero group);
 *            nibble = E2M1_RNE_SAT( R / X ); no per-channel scale (v_scales = 1)
 *   K, Q     one scale per 128-row block: s = amax/448, code = E4M3(x*(448/amax));
 *            K blocks are in permuted order, Q blocks in original order.
 *
 * Q          bf16 [B,H,N,128] or NULL (then q_codes/q_scales are not written)
 * K, V       bf16 [B,H,N,128];  perm int32 [B,H,N] from vc_vsmooth_group
 * q_codes    out u8 [B,H,Np,128] (original order);  q_scales out fp32 [B,H,nb]
 * k_codes    out u8 [B,H,Np,128] (permuted order);  k_scales out fp32 [B,H,nb]
 * v_codes    out, E4M3: u8 [B,H,nb,128(channel),128(row in block)] -- each
 *            block is stored transposed: the code of permuted row 128*t+u,
 *            channel c sits at byte ((bh*nb + t)*128 + c)*128 + u.
 *            NVFP4: u8 [B,H,nb,128(channel),64]: byte ((bh*nb+t)*128+c)*64 + u/2
 *            holds rows u (low nibble, u even) and u+1 (high nibble).
 *            MXFP4: u8 [B,H,nb,128(channel),64]: the 16 bytes at 32h + 16g hold
 *            group (h, g), nibble j (byte j/2, low nibble first) = row 64h+16g+j
 *            for j < 16 and row 64h+32+16g+(j-16) for j >= 16.
 * v_scales   out, E4M3: fp32 [B,H,128] (sv); NVFP4: fp32 [B,H] (St); MXFP4: fp32 [B,H,128] = 1
 * v_group_scales  out, NVFP4: u8 [B,H,Np/16,128] E4M3 scale codes; MXFP4: u8
 *            [B,H,nb,128(channel),2(g),2(h)] E8M0 codes; NULL for E4M3
 * v_means    out bf16 [B,H,nb,128]
 * ------------------------------------------------------------------------ */
size_t vc_preprocess_workspace(int B, int H, int N, int d, int v_format);
int vc_preprocess_quant(const uint16_t* Q, const uint16_t* K, const uint16_t* V, const int32_t* perm,
                        int B, int H, int N, int d, int v_format,
                        uint8_t* q_codes, float* q_scales, uint8_t* k_codes, float* k_scales,
                        uint8_t* v_codes, float* v_scales, uint8_t* v_group_scales,
                        uint16_t* v_means, void* workspace, size_t workspace_bytes, void* stream);

/* vc_preprocess_quant for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and outputs, with no workspace argument.  Its scratch (the
 * residual amax accumulators, vc_preprocess_workspace() bytes) lives in a
 * fixed device array of vc_preprocess_noalloc_max_scratch() = 1 MiB per GPU,
 * reserved by the library for the life of the process and cleared by every
 * call; so B*H <= 2048 for VC_V_E4M3 / VC_V_MXFP4 (VC_V_NVFP4 needs B*H floats
 * only), else VC_ERR_SCRATCH (checked before anything is enqueued).  The
 * first call on a device looks up the array's address on that device (no
 * allocation).  Every call on one GPU shares that array: calls that overlap in
 * time on one GPU (different streams or threads) race and must be serialised
 * by the caller.  Other arguments, outputs and errors as in vc_preprocess_quant. */
size_t vc_preprocess_noalloc_max_scratch(void);
int vc_preprocess_quant_noalloc(const uint16_t* Q, const uint16_t* K, const uint16_t* V, const int32_t* perm,
                                int B, int H, int N, int d, int v_format,
                                uint8_t* q_codes, float* q_scales, uint8_t* k_codes, float* k_scales,
                                uint8_t* v_codes, float* v_scales, uint8_t* v_group_scales,
                                uint16_t* v_means, void* stream);

/* vc_preprocess_quant with the two Q/K steps the pages also fuse into the
 * quantisation kernel (paper digest, preprocessing paragraph: RoPE and a
 * Hadamard transform sit in the same kernel as mean, gather and quantisation;
 * results paragraph: a Hadamard on Q and K moves PSNR by 0.1-0.3 dB at most).
 * The pages define neither; the arithmetic read here, in fp32, row by row:
 *   RoPE      rope_cs: fp32 [N, 64, 2] (cos, sin) per original token position and
 *             channel pair (2i, 2i+1), shared by every (b, h); NULL = no RoPE.
 *             y_2i = fmaf(x_2i, c, -(x_2i+1 * s)), y_2i+1 = fmaf(x_2i, s, x_2i+1 * c)
 *             (inner products rounded once).  A K row uses its token's own
 *             position (before the permutation).
 *   Hadamard  hadamard = 1: y = H y, H the unnormalised 128x128 Sylvester
 *             matrix, computed stage by stage (h = 1, 2, ..., 64; the pair
 *             (i, i+h) with i & h == 0 becomes (a+b, a-b)); K rows are then
 *             multiplied by 2^-7, so Q'.K' = Q.K in real arithmetic.  0 = none.
 * Order: RoPE, Hadamard, then the per-block E4M3 of Q and K as above.  V is not
 * transformed.  hadamard outside {0, 1} -> VC_ERR_INVALID_ARG.  Every other
 * argument and output as in vc_preprocess_quant, which equals this call with
 * rope_cs = NULL and hadamard = 0. */
int vc_preprocess_quant_ex(const uint16_t* Q, const uint16_t* K, const uint16_t* V, const int32_t* perm,
                           int B, int H, int N, int d, int v_format, const float* rope_cs, int hadamard,
                           uint8_t* q_codes, float* q_scales, uint8_t* k_codes, float* k_scales,
                           uint8_t* v_codes, float* v_scales, uint8_t* v_group_scales,
                           uint16_t* v_means, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Non-causal low-bit flash attention with block-mean restore (paper digest,
 * V-Smooth paragraph: each block's mean returns as one outer product with the
 * row sums that online softmax keeps anyway, without a second pass over V;
 * ExpCast-FP8 paragraph for VC_P_EXPCAST).
 *
 * For every query row i (original order) and KV block t (permuted order,
 * ascending -- P codes depend on the running max):
 *   S     = sum_c dec(q_ic) dec(k_jc)           (FP8 MFMA, fp32 accumulate)
 *   kap   = fp32(fp32(sq_i * sk_t) * c0),  c0 = fp32(softmax_scale * log2 e)
 *   mx'   = max(mx, fp32(max_j S * kap))
 *   P     = ExpCast / exp2 codes of S (see vc_p_mode); keys >= N contribute 0
 *   l     = 2^(mx-mx') l + sum_j dec(P)
 *   U     = 2^(mx-mx') U + sum_j dec(P) dec(v_j) + (sum_j dec(P)) mean_t
 *   O     = U / l  (per-channel V scales applied)
 * In the E4M3 and MXFP4 kernels the mean term is added four blocks at a time
 * by a bf16 MFMA with each factor split into a bf16 pair (relative error of the
 * term below 2^-16; everything else as written).
 * Supported pairings: (EXPCAST | FP32EXP_E4M3) with VC_V_E4M3 or VC_V_MXFP4
 * (P.V through the block-scaled FP4 MFMA, the E8M0 group scales applied by the
 * instruction; v_group_scales required), FP32_BF16 with VC_V_NVFP4.  Inputs are
 * the outputs of vc_preprocess_quant (same layouts).
 * out        fp32 [B,H,N,128], original query order
 * ------------------------------------------------------------------------ */
int vc_attn_fp8_fwd(const uint8_t* q_codes, const float* q_scales,
                    const uint8_t* k_codes, const float* k_scales,
                    const uint8_t* v_codes, const float* v_scales, const uint8_t* v_group_scales,
                    const uint16_t* v_means, int B, int H, int N, int d, float softmax_scale,
                    int p_mode, int v_format, float* out, void* stream);

/* ------------------------------------------------------------------------
 * Comparator: standard non-causal flash attention in bf16 (the pages quote all
 * speed-ups against BF16 FlashAttention-4: insight article, section "A Faster
 * Kernel Does Not Automatically Mean Faster Generation"; this is the in-repo
 * stand-in).  bf16 MFMA for Q.K^T and P.V, online softmax with fp32 exp2, P
 * rounded to bf16.  The call first writes V transposed per 128-key block into
 * the workspace (one HBM pass), then runs the attention kernel.
 * Q, K, V    bf16 [B,H,N,128];  out fp32 [B,H,N,128]
 * workspace  device scratch of at least vc_attn_bf16_workspace() bytes
 * ------------------------------------------------------------------------ */
size_t vc_attn_bf16_workspace(int B, int H, int N, int d);
int vc_attn_bf16_fwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int B, int H, int N,
                     int d, float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                     void* stream);

/* ------------------------------------------------------------------------
 * Test hook: vc_attn_fp8_fwd that also records, for every query row and every
 * padded key slot, the fp32 score S and the P byte the kernel fed to the P.V
 * product (E4M3 modes only).  s_dump fp32 [B,H,N,Np], p_dump u8 [B,H,N,Np],
 * key index in permuted order; masked slots get S = 0, P = 0.  Meant for small N
 * (the dumps are N*Np per head).
 * ------------------------------------------------------------------------ */
int vc_attn_fp8_fwd_dump(const uint8_t* q_codes, const float* q_scales,
                         const uint8_t* k_codes, const float* k_scales,
                         const uint8_t* v_codes, const float* v_scales, const uint16_t* v_means,
                         int B, int H, int N, int d, float softmax_scale, int p_mode,
                         float* out, float* s_dump, uint8_t* p_dump, void* stream);

/* ------------------------------------------------------------------------
 * Test hook for every attention pairing: vc_attn_fp8_fwd that also records,
 * for every query row and every padded key slot, the fp32 score S and the P
 * value the kernel fed to its P.V product.  p_dump holds u8 E4M3 codes
 * [B,H,N,Np] for VC_P_EXPCAST / VC_P_FP32EXP_E4M3 (V in VC_V_E4M3 or
 * VC_V_MXFP4) and uint16 bf16 bit patterns [B,H,N,Np] for VC_P_FP32_BF16 (V in
 * VC_V_NVFP4).  s_dump fp32 [B,H,N,Np]; key index in permuted order; masked
 * slots get S = 0, P = 0.  Other arguments, outputs and errors as in
 * vc_attn_fp8_fwd.  Meant for small N (the dumps are N*Np per head).
 * ------------------------------------------------------------------------ */
int vc_attn_fwd_dump(const uint8_t* q_codes, const float* q_scales,
                     const uint8_t* k_codes, const float* k_scales,
                     const uint8_t* v_codes, const float* v_scales, const uint8_t* v_group_scales,
                     const uint16_t* v_means, int B, int H, int N, int d, float softmax_scale,
                     int p_mode, int v_format, float* out, float* s_dump, void* p_dump, void* stream);

/* ------------------------------------------------------------------------
 * Test hook: one gfx950 instruction on caller data, so that tests can record
 * the device facts the kernels rely on (element counts n; all device memory):
 *   what 0  V_CVT_PK_FP8_F32, no clamp first   in fp32 [n] -> out u8 [n]
 *   what 1  V_CVT_PK_U8_F32                     in fp32 [n] -> out u8 [n]
 *   what 2  V_EXP_F32                           in fp32 [n] -> out fp32 [n]
 *   what 3  V_MFMA_F32_32X32X64_F8F6F4, E4M3    n tiles: in = A u8 [32][64],
 *           B u8 [32][64], C fp32 [32][32] per tile; out D fp32 [32][32] per
 *           tile, D = A . B^T + C
 *   what 4  V_MFMA_F32_16X16X128_F8F6F4, E4M3   the same with 16, 16, 128
 * and three HBM streams over n 16-byte words (2048 workgroups x 256 threads):
 *   what 5  read only                           in [n] -> out u32 [2048*256]
 *   what 6  copy                                in [n] -> out [n]
 *   what 7  two reads per write                 in [2n] -> out [n], out[i] = in[i] ^ in[i+n]
 * and the FP8 MFMA throughput:
 *   what 8  n workgroups x 4 wavefronts, each 2048 x 4 independent
 *           V_MFMA_F32_32X32X64_F8F6F4 on operands from in (u8 [2048])
 *                                               -> out fp32 [n*256] (accumulator sums)
 * and the vector-instruction issue rate:
 *   what 9  n workgroups x 8 wavefronts (one workgroup per CU), in = i32 [2]
 *           {instruction: 0 V_FMA_F32, 1 V_EXP_F32; wavefronts running it:
 *           4 = one per SIMD, 8 = two}, each running wavefront 4096 x 8
 *           independent chains   -> out i64 [n*8][2] (s_memtime ticks of the
 *           loop, 0 when idle; bits of the lane-0 chain sum)
 * and the rate of the global -> LDS tile copies:
 *   what 10 n workgroups x 8 wavefronts (one workgroup per CU), in = u8
 *           [256 + 8192]: i32 {mode, iterations} then an 8 KiB source; each
 *           iteration a wavefront issues eight 64-lane loads of the source and
 *           waits: mode 0 16 bytes per lane into LDS, 1 4 bytes per lane into
 *           LDS, 2 16 bytes per lane into registers
 *                                               -> out i64 [n*8][2] (s_memtime ticks of the
 *           loop; a checksum of the loaded data)
 * Returns VC_ERR_UNSUPPORTED for other `what`, VC_ERR_INVALID_ARG for null
 * pointers or n < 1.
 * ------------------------------------------------------------------------ */
int vc_device_probe(int what, const void* in, void* out, int n, void* stream);

/* ------------------------------------------------------------------------
 * Grouping cadence over a denoising trajectory (paper digest, clustering-
 * rationale paragraph and limitations; news article, "V-Smooth"; insight
 * article, "Value Is the Error Source Earlier Methods Underestimated"): grouping
 * runs only during the first quarter of the denoising steps, and each
 * permutation serves four adjacent steps.  Host-only calls; no GPU work.
 *
 * Reading: step s (0-based, 0 <= s < total_steps) lies in the grouping window
 * when s < fraction * total_steps (as real numbers); a step in the window
 * regroups when s % reuse == 0, so step 0 always regroups.  Every step uses the
 * permutation of the latest regrouping step at or before it; steps past the
 * window keep the last one.  The pages' cadence is reuse = 4, fraction = 0.25.
 *
 * vc_group_due     1 if step s computes a new permutation, 0 if it reuses one
 * vc_group_source  the step whose permutation step s uses
 * vc_group_count   regrouping steps over the whole trajectory
 * Each returns VC_ERR_INVALID_ARG when total_steps < 1, step is outside
 * [0, total_steps), reuse < 1 or fraction is outside (0, 1].
 * ------------------------------------------------------------------------ */
int vc_group_due(int step, int total_steps, int reuse, float fraction);
int vc_group_source(int step, int total_steps, int reuse, float fraction);
int vc_group_count(int total_steps, int reuse, float fraction);

const char* vc_status_string(int status);
int vc_last_hip_error(void);
const char* vc_version(void);

#ifdef __cplusplus
}
#endif
#endif /* VC_ATTN_VC_H */
