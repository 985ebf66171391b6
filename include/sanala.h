/*
 * libsanala -- ReLU linear self-attention with QK-RMSNorm for AMD Instinct MI355X (gfx950).
 *
 * The operation (per sample b, head h, token i), from "Sana: Efficient High-Resolution Image
 * Synthesis with Linear Diffusion Transformers" (paper notes), section 2.1 "linear attention",
 * Eq. (1), with the QK Norm of "SANA 1.5: Efficient Scaling of Training-Time and Inference-Time
 * Compute in Linear Diffusion Transformer" (research notes), section "model architecture":
 *
 *   phi(x)   = ReLU( x / sqrt(mean_c x_c^2 + eps) * g )     RMSNorm over all C = H*D channels
 *   S_h      = sum_j phi(K_j,h)^T V_j,h                      D x D, accumulated in fp32
 *   z_h      = sum_j phi(K_j,h)                              D, fp32
 *   O_i,h    = phi(Q_i,h) S_h / ( phi(Q_i,h) . z_h + eps )
 *
 * The sum over j is over all N tokens of the sample (non-causal).  Head h owns channels
 * [h*D, (h+1)*D) of a token row.  The same eps is added inside the RMSNorm square root and to the
 * attention denominator.  Passing gq = gk = NULL switches the QK-Norm off: phi(x) = ReLU(x).
 *
 * Layout: every token tensor is row-major [B, N, C] with C = H*D contiguous channels per token;
 * gq and gk are fp32 [C].  All tensor pointers are device pointers owned by the caller; the
 * library never frees or keeps them.  `out` must not overlap any input.
 *
 * Calls are asynchronous on `stream` and return without a host synchronisation.  Argument checks
 * happen on the host before anything is enqueued; faults inside kernels surface at the caller's
 * next synchronisation.  NaN/Inf in the inputs propagate to the outputs they touch; nothing checks
 * for them.
 *
 * Scratch memory (row statistics, split-N partial states, the reduced state, and for the fused calls
 * the qkv buffer) is owned by the library: one buffer per (device, stream), taken from the device's
 * stream-ordered pool with hipMallocAsync on `stream` the first time and reused by later calls on the
 * same stream (stream order runs them after the earlier calls' kernels); a call that needs more frees
 * it on `stream` and takes a larger one.  Calls on different streams never share scratch; calls from
 * several host threads on one stream are serialised while they enqueue.  There is no limit on the
 * number of streams.  A buffer is kept until sana_release_scratch(stream) frees it (call that before
 * destroying a stream the library has used) or the process ends.  Every call records an event on its
 * stream after its work, and the next call on the same buffer makes its stream wait for that event
 * unless it has completed: if a stream is destroyed without sana_release_scratch and the runtime hands
 * its handle value to a new stream, the new stream's calls still start only after the old kernels
 * that used the buffer have finished.
 * Results are bitwise reproducible: every reduction runs in a fixed order, with no floating-point
 * atomics.
 */
#ifndef SANALA_H
#define SANALA_H

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SANA_OK = 0,
  SANA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad eps, only one gain NULL, ... */
  SANA_ERR_UNSUPPORTED = 2, /* a shape or dtype the library has no kernel for (D != 32, ...) */
  SANA_ERR_MISALIGNED = 3,  /* a tensor pointer is not 16-byte aligned */
  SANA_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  SANA_ERR_SCRATCH_LIMIT = 5 /* sana_linear_attn_fwd_noalloc: the call needs more than its static scratch */
} sana_status_t;

typedef enum {
  SANA_F32 = 0,  /* fp32 storage, fp32 arithmetic */
  SANA_BF16 = 1, /* bf16 storage; fp32 accumulation; bf16 MFMA operands; outputs rounded to nearest even */
  SANA_F16 = 2   /* IEEE binary16 storage; fp32 sums of squares and KV state (fp16 MFMA operands for the
                    state, bf16 operands for the output contraction, whose state values can exceed
                    the binary16 range); outputs rounded to nearest even (overflow gives +-inf) */
} sana_dtype_t;

/*
 * sana_linear_attn_fwd -- O = linear attention of (q, k, v) as defined above.
 *
 *   q, k, v  device, [B, N, H*D] of `dtype`, contiguous, 16-byte aligned.
 *   gq, gk   device, fp32 [H*D]: RMSNorm gains of Q and K; both NULL for QK-Norm off.
 *   B, N, H  >= 1; D must be 32.  B*N*H*D < 2^40.
 *   eps      finite, >= 0 (SANA uses 1e-6).
 *   out      device, [B, N, H*D] of `dtype`, contiguous, 16-byte aligned; fully overwritten.
 *   stream   HIP stream the work is enqueued on (0 = the null stream).
 *   dtype    SANA_F32, SANA_BF16 or SANA_F16 (storage type of q, k, v and out).
 *
 * Returns SANA_OK once the work is enqueued, or an error code with nothing enqueued.
 */
sana_status_t sana_linear_attn_fwd(const void* q, const void* k, const void* v,
                                   const float* gq, const float* gk,
                                   int B, int N, int H, int D, float eps,
                                   void* out, hipStream_t stream, sana_dtype_t dtype);

/*
 * sana_linear_attn_fwd_noalloc -- sana_linear_attn_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * kernels and results (bit for bit) as sana_linear_attn_fwd; the scratch is a static device array of
 * 64 MiB per GPU, part of the library's code object, which each GPU the library runs on holds until the
 * process ends.  The call itself allocates nothing: no hipMalloc, hipFree or stream-ordered pool use,
 * and no timing events (sana_timing_enable does not apply to it).  The caller still passes q, k, v,
 * gains and out.
 *
 * A call whose scratch exceeds 64 MiB returns SANA_ERR_SCRATCH_LIMIT with nothing enqueued (the
 * 16384-token and the 32 x 1024-token workloads need about 4.4 and 5.0 MB).  Every call on a GPU
 * shares that GPU's array and leaves its contents behind; nothing in it has to start at any value (each
 * kernel writes every element it later reads).  Calls that overlap on one GPU (on different streams,
 * or from several host threads without ordering) race on the array and give undefined results:
 * serialise them, e.g. on one stream.  Errors otherwise as for sana_linear_attn_fwd.
 */
sana_status_t sana_linear_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                                           const float* gq, const float* gk,
                                           int B, int N, int H, int D, float eps,
                                           void* out, hipStream_t stream, sana_dtype_t dtype);

/*
 * sana_qkv_linear_attn_fwd -- fused front end: qkv = x @ Wqkv (bf16 MFMA GEMM, fp32 accumulation,
 * qkv rounded to bf16), then sana_linear_attn_fwd on the q | k | v column blocks.  The QKV
 * projection is the one the Sana notes (section 7, on-device deployment) fuse with ReLU(K)^T V.
 *
 *   x        device bf16 [B, N, C], C = H*D, contiguous, 16-byte aligned.
 *   Wqkv     device bf16 [C, 3C] row-major (x @ Wqkv); columns [0,C) give q, [C,2C) k, [2C,3C) v;
 *            no bias.
 *   gq, gk   device fp32 [C], or both NULL (QK-Norm off).
 *   B, N, H  >= 1; D must be 32.
 *   eps      finite, >= 0.
 *   out      device bf16 [B, N, C]; fully overwritten.
 *   stream   HIP stream.
 *
 * The qkv intermediate (B*N*3C bf16) and a copy of x laid out for the projection GEMM live in the
 * stream's scratch.  Errors as above.
 */
sana_status_t sana_qkv_linear_attn_fwd(const void* x, const void* Wqkv,
                                       const float* gq, const float* gk,
                                       int B, int N, int H, int D, float eps,
                                       void* out, hipStream_t stream);

/*
 * sana_pack_weight_i8 -- lays out a quantised weight for sana_qkv_w8a8_linear_attn_fwd (done once per
 * weight, e.g. when a model is loaded).  Wt_q [rows, C] row-major becomes K-blocked: byte
 * ((c / 64) * rows + n) * 64 + c % 64 of Wt_p holds Wt_q[n, c], so every 64-channel slice of all rows is
 * one contiguous run.  A pure copy: the codes are not changed.
 *
 *   Wt_q     device int8 [rows, C] row-major, 16-byte aligned.
 *   rows     >= 1, <= 2^30;  C >= 1, a multiple of 64;  rows * C <= 2^40 (else SANA_ERR_UNSUPPORTED).
 *   Wt_p     device int8, rows * C bytes, 16-byte aligned, not overlapping Wt_q; fully overwritten.
 *
 * Returns SANA_OK once enqueued on `stream`; argument errors as above.
 */
sana_status_t sana_pack_weight_i8(const void* Wt_q, int64_t rows, int C, void* Wt_p, hipStream_t stream);

/*
 * sana_qkv_w8a8_linear_attn_fwd -- the fused front end with the projection in W8A8 (the Sana notes,
 * section 7: 8-bit weights and activations for deployment, with the linear attention kept in full
 * precision).  x is quantised per token on the device (sana_quantize_rows_i8), the projection runs on
 * int8 MFMA with exact int32 sums, qkv = bf16((sum_c xq[m,c] * Wt_q[n,c]) * x_scale[m] * w_scale[n])
 * (fp32 products in that order), and the attention is that of sana_linear_attn_fwd on bf16 q | k | v.
 *
 *   x        device bf16 [B, N, C], C = H*D, contiguous, 16-byte aligned.
 *   Wt_p     device int8, 3C * C bytes: sana_pack_weight_i8(Wt_q, 3C, C, Wt_p) of the quantised weight
 *            transposed, Wt_q [3C, C], row n holding the C input weights of output column n (q = rows
 *            [0,C), k = [C,2C), v = [2C,3C)); 16-byte aligned.
 *   w_scale  device fp32 [3C]: dequantisation scale of each output column (W[:, n] ~ w_scale[n] *
 *            Wt_q[n, :]); 16-byte aligned.  The scale granularity is a reading: the pages do not fix it.
 *   gq, gk, B, N, H, D, eps, out, stream as for sana_qkv_linear_attn_fwd; C must be a multiple of 64
 *            (else SANA_ERR_UNSUPPORTED).
 *
 * Scratch (the stream's buffer): int8 x, its row scales and the bf16 qkv.  Errors as above.
 */
sana_status_t sana_qkv_w8a8_linear_attn_fwd(const void* x, const void* Wt_p, const float* w_scale,
                                            const float* gq, const float* gk,
                                            int B, int N, int H, int D, float eps,
                                            void* out, hipStream_t stream);

/*
 * sana_mix_ffn_fwd -- Mix-FFN, the feed-forward half of the Linear DiT block (the Sana notes, section
 * 2.2: inverted residual block, 3x3 depthwise convolution, GLU; section 2.3: zero padding of that
 * convolution):  h = x @ W1 (bf16 MFMA GEMM, rounded to bf16); u = 3x3 depthwise cross-correlation
 * of h over each sample's Hg x Wg token grid with zero padding; g = u[:, :F] * sigmoid(u[:, F:])
 * (fp32, rounded to bf16); out = g @ W2 (bf16 GEMM).  No biases; the block's residual add is the
 * caller's.
 *
 *   x        device bf16 [B, Hg*Wg, C], tokens in raster order (n = i*Wg + j), 16-byte aligned.
 *   W1       device bf16 [C, 2F] row-major: columns [0,F) the values, [F,2F) the gates.
 *   Wdw      device bf16 [2F, 3, 3]: tap (p, q) of channel c reads grid row i+p-1, column j+q-1.
 *   W2       device bf16 [F, C] row-major.
 *   B, Hg, Wg  >= 1, Wg <= 128; C and F multiples of 32, at most 2^20 (SANA: C = 2240, F = 5600).
 *   out      device bf16 [B, Hg*Wg, C], 16-byte aligned, not overlapping the inputs; fully overwritten.
 *
 * Scratch (the stream's buffer): h (B*Hg*Wg*2F bf16) and B*Hg*Wg*max(C, F) bf16 for a copy of x laid out
 * for the expansion GEMM, later reused for g.  Errors as above.
 */
sana_status_t sana_mix_ffn_fwd(const void* x, const void* W1, const void* Wdw, const void* W2,
                               int B, int Hg, int Wg, int C, int F, void* out, hipStream_t stream);

/*
 * sana_cross_attn_fwd -- the Linear DiT block's cross-attention with QK-Norm ("SANA 1.5: Efficient
 * Scaling of Training-Time and Inference-Time Compute in Linear Diffusion Transformer", research
 * notes, model architecture: vanilla cross-attention injecting the text condition; QK Norm on its
 * queries and keys).  Per sample b, head h (channels [32h, 32h+32)) and image token i:
 *   qn = q * r_q * gq, kn = k * r_k * gk with r = 1/sqrt(mean over all C channels of x^2 + eps);
 *   o[b,i,h] = sum_j softmax_j(qn[b,i,h] . kn[b,j,h] / sqrt(D)) v[b,j,h] over the text tokens
 *   j < kv_len[b].  NULL gains: the norm is off.  The projections around it are the caller's.
 *
 *   q        device bf16 [B, N, C] image-token queries, C = H*D, contiguous, 16-byte aligned.
 *   k, v     device bf16 [B, L, C] text-token keys and values, contiguous, 16-byte aligned.
 *   gq, gk   device fp32 [C] RMSNorm gains, 16-byte aligned, or both NULL.
 *   kv_len   device int32 [B]: valid text tokens of each sample (the rest is padding), or NULL for
 *            all L.  Read on the device, so not checked: values are clamped to [0, L], and a sample with
 *            0 valid tokens gets an all-zero output.
 *   B >= 1 (<= 65535), N >= 1, 1 <= L <= 1024, D == 32, 1 <= H <= 128 (else SANA_ERR_UNSUPPORTED).
 *   eps      finite, >= 0.
 *   out      device bf16 [B, N, C], 16-byte aligned, not overlapping q, k or v; fully overwritten.
 *   dtype    SANA_BF16 (others: SANA_ERR_UNSUPPORTED).
 *
 * Arithmetic: fp32 statistics; with the norm the keys enter the MFMA as bf16(k * r_k * gk) and the
 * queries as bf16(q * r_q * gq * log2(e)/sqrt(D)) (the softmax scale taken into that one rounding), and
 * the subtracted constant is added on the MFMA as a bf16 pair; without the norm q and k enter as given
 * and the scale and constant are applied in fp32.  Logits are fp32 sums of the exact bf16 products, the
 * softmax in fp32 (exp2), the softmax weights rounded to bf16 for the value product, fp32 accumulation,
 * bf16 output (round to nearest even).
 * Scratch (the stream's buffer): the normalised keys (B*L*C bf16) and r_q (B*N fp32).  Errors as above.
 */
sana_status_t sana_cross_attn_fwd(const void* q, const void* k, const void* v, const float* gq, const float* gk,
                                  const int* kv_len, int B, int N, int L, int H, int D, float eps, void* out,
                                  hipStream_t stream, sana_dtype_t dtype);

/*
 * sana_quantize_rows_i8 -- per-row symmetric int8 quantisation of bf16 x [rows, C] (the activation
 * half of W8A8): with a = max_c |x[r, c]|, xq = clamp(rne(x * (127 / a)), -127, 127) and
 * x_scale[r] = a / 127, each step in fp32 with correctly rounded division; a row of zeros gives
 * xq = 0 and x_scale = 0.  NaN inputs are not checked.
 *
 *   x        device bf16 [rows, C], contiguous, 16-byte aligned; C a multiple of 8, rows <= 2^32.
 *   xq       device int8 [rows, C], 16-byte aligned, not overlapping x; fully overwritten.
 *   x_scale  device fp32 [rows]; fully overwritten.
 *
 * Returns SANA_OK once enqueued on `stream`; argument errors as above.
 */
sana_status_t sana_quantize_rows_i8(const void* x, int64_t rows, int C, void* xq, float* x_scale,
                                    hipStream_t stream);

/*
 * sana_release_scratch -- frees the library's scratch buffer of `stream` on the current device,
 * stream-ordered (hipFreeAsync on `stream`, so kernels already queued on it finish first), and forgets
 * the stream.  `stream` must still exist.  A later call on `stream` takes a new buffer.  Returns
 * SANA_OK (also when the stream has no buffer) or SANA_ERR_HIP if the free fails.
 */
sana_status_t sana_release_scratch(hipStream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* sana_status_string(sana_status_t status);

/*
 * Measurement support for benchmarks and profilers (not part of the method).
 *
 * sana_timing_enable(1) makes every later call from the calling host thread launch each kernel with a
 * start/stop HIP event pair that the kernel's own dispatch timestamps (hipExtLaunchKernelGGL), so the
 * durations are the kernels' own; sana_timing_enable(0) stops it.  Events are created once per thread
 * and reused.  Timing adds a little host overhead per launch, so throughput runs leave it off.
 *
 * sana_timing_last waits for the events of the most recent call on this thread and writes, for up
 * to `capacity` kernels in launch order, a static kernel name (names may be NULL) and the kernel's
 * duration in milliseconds (ms may be NULL; -1 if an event failed).  Returns the number of kernels
 * that call launched.
 */
sana_status_t sana_timing_enable(int enable);
int sana_timing_last(const char** names, float* ms, int capacity);

#ifdef __cplusplus
}
#endif

#endif /* SANALA_H */
