/*
 * mt_ops.h - the kernels of the streamed training step, one entry point each.
 *
 * mt_train_step (mt.h) runs these same kernels in its layer template. They are
 * exported so that each kernel can be checked and timed on its own. Device
 * pointers are device memory the caller owns; `stream` is a hipStream_t passed
 * as void* (NULL = the null stream). Launches are asynchronous on `stream`.
 * Return 0, or MT_EINVAL for unsupported shapes, dtypes or NULL pointers
 * (checked on the host before any launch), or MT_EHIP if a launch fails.
 * dtype arguments are MT_FP32 or MT_BF16 (mt.h); a `void*` operand of dtype
 * MT_BF16 holds bfloat16 values (round-to-nearest-even from fp32).
 *
 * Every layout is row-major. M = B*T tokens in (b, t) order.
 */
#ifndef MT_OPS_H
#define MT_OPS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MT_GEMM_NT 0  /* C[M,N] = A[M,K] . B[N,K]^T   (Linear forward)         */
#define MT_GEMM_NN 1  /* C[M,N] = A[M,K] . B[K,N]     (input gradient dX = dY W) */
#define MT_GEMM_TN 2  /* C[M,N] = A[K,M]^T . B[K,N]   (weight gradient dW = dY^T X) */

/* Matrix product on the matrix cores: A and B both of `dtype`, fp32
 * accumulation, fp32 result C (leading dimension ldc). If R is not NULL,
 * C = R + A.B (R has leading dimension ldr and may alias C). lda/ldb are the
 * leading dimensions of A and B as stored. Any M, N, K >= 0 (K = 0 gives
 * C = R or 0). */
int mt_op_gemm(int32_t dtype, int32_t layout, const void* A, int64_t lda, const void* B,
               int64_t ldb, float* C, int64_t ldc, const float* R, int64_t ldr, int64_t M,
               int64_t N, int64_t K, void* stream);

/* mt_op_gemm with the tile size chosen by the caller: variant 0 = by shape
 * (as mt_op_gemm), 1 = 128x128 tiles, 2 = 256x256 tiles (used when A and B
 * rows are 16-byte aligned; otherwise 128x128). For tests and tuning. */
int mt_op_gemm_variant(int32_t dtype, int32_t layout, const void* A, int64_t lda, const void* B,
                       int64_t ldb, float* C, int64_t ldc, const float* R, int64_t ldr, int64_t M,
                       int64_t N, int64_t K, int32_t variant, void* stream);

/* mt_op_gemm with a device workspace ws of ws_bytes (16-byte aligned; NULL or
 * 0 bytes: no split, as mt_op_gemm). When the 256x256 tiles of the product
 * leave the last wave of workgroups at most half full (or fill at most half
 * of one), those tiles are split along K: the split blocks write partials to
 * ws, and a second kernel adds them to C in a fixed order (deterministic;
 * the rounding differs from the unsplit product by the summation order).
 * mt_op_gemm_ws_bytes() is the size that allows every split. Calls sharing
 * a workspace must be ordered on one stream. */
int64_t mt_op_gemm_ws_bytes(void);
int mt_op_gemm_ws(int32_t dtype, int32_t layout, const void* A, int64_t lda, const void* B, int64_t ldb,
                  float* C, int64_t ldc, const float* R, int64_t ldr, int64_t M, int64_t N, int64_t K,
                  void* ws, int64_t ws_bytes, void* stream);

/* RMSNorm forward over rows of x [rows, d] (fp32): y = x r w with
 * r = (mean(x^2) + eps)^(-1/2), written as out_dtype; rstd[rows] = r. */
int mt_op_rmsnorm_fwd(int32_t out_dtype, const float* x, const float* w, void* y, float* rstd,
                      int64_t rows, int32_t d, float eps, void* stream);

/* RMSNorm backward given dy [rows, d] (fp32): dx = r (dy w - x r^2 mean(dy w x)),
 * written to dx (accumulate != 0: dx += ...), and dw[d] = sum over rows of
 * dy x r, summed in a fixed order. ws: mt_op_rmsnorm_bwd_ws_floats(rows, d)
 * floats of scratch. x, w, dy, dx and ws are read and written 16 bytes at a
 * time and must be 16-byte aligned (MT_EINVAL otherwise). */
int64_t mt_op_rmsnorm_bwd_ws_floats(int64_t rows, int32_t d);
int mt_op_rmsnorm_bwd(const float* x, const float* w, const float* rstd, const float* dy,
                      float* dx, int32_t accumulate, float* dw, float* ws, int64_t rows,
                      int32_t d, void* stream);

/* RoPE table on the host: cos/sin[t][i] of t * base^(-2i/hd), t < T,
 * i < hd/2, computed in double and stored as float (host pointers, T*hd/2). */
int mt_rope_table(int32_t T, int32_t hd, float base, float* cos_out, float* sin_out);

/* Rotary embedding of the packed projection output qkv [M, (H + 2 Hkv) hd]
 * (q heads, then k heads, then v heads; fp32): q and k heads are rotated
 * half-split by angle t * base^(-2i/hd) (t = token position within its
 * sequence), v is copied; written as out_dtype in the same layout.
 * cos/sin: device tables [T][hd/2]. The backward rotates by the negative angle. */
int mt_op_rope_fwd(int32_t out_dtype, const float* qkv, void* out, const float* cos,
                   const float* sin, int32_t B, int32_t T, int32_t H, int32_t Hkv,
                   int32_t hd, void* stream);
int mt_op_rope_bwd(int32_t out_dtype, const float* dqkv, void* out, const float* cos,
                   const float* sin, int32_t B, int32_t T, int32_t H, int32_t Hkv,
                   int32_t hd, void* stream);

/* Causal flash attention forward on the packed, rotated qkv [M, (H+2Hkv) hd]
 * of `dtype`: o [M, H hd] fp32 (and, if o_cast is not NULL, o as `dtype` in
 * o_cast), lse [B, H, T] fp32 = natural-log logsumexp of each row of scaled,
 * masked scores. Scale 1/sqrt(hd); query head h reads kv head h / (H/Hkv). */
int mt_op_attn_fwd(int32_t dtype, const void* qkv, float* o, void* o_cast, float* lse,
                   int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t hd, void* stream);

/* Causal flash attention backward: given qkv (as in forward), o and dout
 * [M, H hd] fp32 and lse, writes dqkv [M, (H+2Hkv) hd] fp32 (dq, then dk and
 * dv summed over each kv group). P is recomputed from lse; D = rowsum(dout o)
 * in fp32; dq and dk/dv come from separate, deterministic passes (in bf16
 * mode with H > Hkv and T <= 8192, dk/dv per query head, then summed over
 * the group in head order). ws: mt_op_attn_bwd_ws_bytes(...) bytes of device
 * scratch. */
int64_t mt_op_attn_bwd_ws_bytes(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t hd);
int mt_op_attn_bwd(int32_t dtype, const void* qkv, const float* o, const float* dout,
                   const float* lse, float* dqkv, void* ws, int32_t B, int32_t T, int32_t H,
                   int32_t Hkv, int32_t hd, void* stream);

/* mt_op_attn_bwd followed by the RoPE backward, in one pass: the q and k
 * gradients are rotated by the negative angle of their position (cos/sin as
 * in mt_op_rope_bwd, [T][hd/2]) and every gradient is written as `dtype`
 * into dqkv [M, (H+2Hkv) hd]: the gradient of the unrotated projection
 * output. Same values as mt_op_attn_bwd then mt_op_rope_bwd(dtype, ...),
 * without the fp32 intermediate. */
int mt_op_attn_bwd_rope(int32_t dtype, const void* qkv, const float* o, const float* dout,
                        const float* lse, const float* cos, const float* sin, void* dqkv,
                        void* ws, int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t hd,
                        void* stream);

/* mt_op_attn_bwd_rope without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Its scratch is a static device array of
 * MT_NOALLOC_SCRATCH_BYTES per GPU, held from library load until the process
 * ends; nothing is allocated or freed by the call. Same kernels, arguments
 * (less ws) and results as mt_op_attn_bwd_rope. MT_EINVAL, with
 * mt_last_error(NULL) stating the need, when mt_op_attn_bwd_ws_bytes(dtype,
 * B, T, H, hd) exceeds MT_NOALLOC_SCRATCH_BYTES (64 MiB: for example the
 * 14B-shaped layer's 40 heads of 128 over 1024 tokens in bf16 mode).
 * Every call on one GPU shares that GPU's scratch and overwrites it: calls
 * that overlap on one GPU (other streams or threads) race; order them on one
 * stream. */
#define MT_NOALLOC_SCRATCH_BYTES (64ll << 20)
int mt_op_attn_bwd_rope_noalloc(int32_t dtype, const void* qkv, const float* o, const float* dout,
                                const float* lse, const float* cos, const float* sin, void* dqkv, int32_t B,
                                int32_t T, int32_t H, int32_t Hkv, int32_t hd, void* stream);

/* SwiGLU on gu [M, 2F] fp32 (gate = columns [0, F), up = [F, 2F)):
 * act = silu(gate) up as out_dtype [M, F]. Backward: from dact [M, F] fp32,
 * dgu [M, 2F] as out_dtype with dgate = dact up s (1 + gate (1 - s)),
 * dup = dact gate s, s = sigmoid(gate). */
int mt_op_swiglu_fwd(int32_t out_dtype, const float* gu, void* act, int64_t M, int32_t F,
                     void* stream);
int mt_op_swiglu_bwd(int32_t out_dtype, const float* gu, const float* dact, void* dgu,
                     int64_t M, int32_t F, void* stream);

/* Cross-entropy over rows of logits [rows, V] fp32 with targets[rows]:
 * loss[r] = logsumexp(z_r) - z_r[target_r]; dlogits = scale (softmax(z_r) -
 * onehot) as out_dtype (may alias logits when out_dtype is MT_FP32). */
int mt_op_xent(int32_t out_dtype, const float* logits, const int32_t* targets, float* loss,
               void* dlogits, int64_t rows, int32_t V, float scale, void* stream);

/* y = x rounded to out_dtype (n elements). */
int mt_op_cast(int32_t out_dtype, const float* x, void* y, int64_t n, void* stream);

/* Host AdamW over n fp32 elements at step count t >= 1 (decoupled decay):
 * p <- p(1 - lr wd); m <- b1 m + (1-b1) g; v <- b2 v + (1-b2) g^2;
 * p <- p - (lr / (1-b1^t)) m / (sqrt(v) / sqrt(1-b2^t) + eps).
 * The step constants are formed in double and applied in fp32 arithmetic.
 * If bf16_out is not NULL it receives bf16(p) (round to nearest even).
 * threads: 0 = online CPUs. */
int mt_adamw_host(float* p, float* m, float* v, const float* g, int64_t n, int64_t t, double lr,
                  double beta1, double beta2, double eps, double weight_decay, uint16_t* bf16_out,
                  int32_t threads);

/* mt_adamw_host with the gradient given as bf16 bit patterns g16[n] (the
 * MT_BF16_GRADS transfer format), widened exactly to fp32 before the same
 * update; if g32_out is not NULL it receives the widened gradient. */
int mt_adamw_host_g16(float* p, float* m, float* v, const uint16_t* g16, float* g32_out, int64_t n, int64_t t,
                      double lr, double beta1, double beta2, double eps, double weight_decay,
                      uint16_t* bf16_out, int32_t threads);

#ifdef __cplusplus
}
#endif

#endif /* MT_OPS_H */
