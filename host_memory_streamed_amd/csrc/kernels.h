// Host-side launchers of the gfx950 kernels (defined in the .hip files).
// Plain types only, so host translation units compiled with g++ can call them.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "mt_ops.h"

namespace mt {

// dtype: 0 = fp32, 1 = bf16 (same values as MT_FP32 / MT_BF16)
hipError_t gemm(int dtype, int layout, const void* A, int64_t lda, const void* B, int64_t ldb,
                float* C, int64_t ldc, const float* R, int64_t ldr, int64_t M, int64_t N,
                int64_t K, hipStream_t s);
// variant: 0 = choose by shape, 1 = 128x128 tiles, 2 = 256x256 tiles (when aligned)
hipError_t gemm_variant(int dtype, int layout, const void* A, int64_t lda, const void* B, int64_t ldb,
                        float* C, int64_t ldc, const float* R, int64_t ldr, int64_t M, int64_t N,
                        int64_t K, int variant, hipStream_t s);
// As gemm; with a device workspace of ws_bytes (GEMM_WS_BYTES enables every
// split), the tiles of a last, at most half-full wave of 256x256 workgroups
// are split along K and their partials added in a fixed order. Calls that
// share a workspace must be ordered (one stream).
constexpr int64_t GEMM_WS_BYTES = 64ll << 20;
hipError_t gemm_ws(int dtype, int layout, const void* A, int64_t lda, const void* B, int64_t ldb, float* C,
                   int64_t ldc, const float* R, int64_t ldr, int64_t M, int64_t N, int64_t K, void* ws,
                   int64_t ws_bytes, hipStream_t s);

// Limits set by the kernels' 32-bit quantities. Work-items per grid dimension
// stay below 2^32: the kernels that give each row a 256-thread block (RoPE,
// cross-entropy) take fewer than MAX_BLOCK_ROWS rows. Every element index that
// involves the token count is 64-bit. The direct global->LDS copies address
// their bytes as a 32-bit offset from a 64-bit tile base: attention tiles span
// 64 rows of the packed projection, (H + 2 Hkv) hd elements each, so that row
// length stays below MAX_ATTN_LD; GEMM tiles span 256 rows of an operand, and
// operands with longer rows take the 128x128 kernel, which loads through
// 64-bit pointers.
constexpr int64_t MAX_BLOCK_ROWS = 1ll << 24;
constexpr int64_t MAX_ATTN_LD = 1ll << 24;
constexpr int64_t MAX_COPY_OFFSET = 1ll << 31;

bool attn_supported(int dtype, int hd);
// bf16 forward on 32x32 matrix-core tiles (hd 64 or 128), attn_fwd_bf16.hip
hipError_t attn_fwd_bf16(const void* qkv, float* o, void* o_cast, float* lse, int B, int T, int H,
                         int Hkv, int hd, hipStream_t s);
// bf16 backward on 32x32 matrix-core tiles (hd 64 or 128), attn_bwd_bf16.hip;
// arguments as attn_bwd
hipError_t attn_bwd_bf16(const void* qkv, const float* o, const float* dout, const float* lse, void* dqkv,
                         int out_dtype, const float* rcos, const float* rsin, void* ws, int B, int T, int H,
                         int Hkv, int hd, hipStream_t s);
int64_t attn_ws_d_bytes(int B, int T, int H);
// bf16 attention backward: head subsets per dK/dV work item (attn_bwd_bf16.hip)
// and the workspace its fp32 partials take
int attn_dkv_hsplit(int Tn, int H, int Hkv);
int64_t attn_dkv_part_bytes(int B, int Tn, int H, int hd);
hipError_t attn_fwd(int dtype, const void* qkv, float* o, void* o_cast, float* lse, int B, int T,
                    int H, int Hkv, int hd, hipStream_t s);
// dqkv of out_dtype (fp32, or bf16 when dtype is bf16); with rcos/rsin (the
// RoPE tables) the q and k gradients are rotated back to the unrotated
// projection output, else they are the gradients of the rotated operands.
hipError_t attn_bwd(int dtype, const void* qkv, const float* o, const float* dout, const float* lse,
                    void* dqkv, int out_dtype, const float* rcos, const float* rsin, void* ws, int B,
                    int T, int H, int Hkv, int hd, hipStream_t s);

int rmsnorm_bwd_partials(int64_t rows);
hipError_t rmsnorm_fwd(int out_dtype, const float* x, const float* w, void* y, float* rstd,
                       int64_t rows, int d, float eps, hipStream_t s);
// dx written (accumulate 0) or added to; dw written (dw_accumulate 0) or added to
hipError_t rmsnorm_bwd(const float* x, const float* w, const float* rstd, const float* dy,
                       float* dx, int accumulate, float* dw, float* ws, int64_t rows, int d,
                       hipStream_t s, int dw_accumulate = 0);
// rows [row0, row0 + rows) of the token sequence (positions (row0 + i) % T);
// `in` and `out` point at the first of those rows
hipError_t rope(int out_dtype, int backward, const float* in, void* out, const float* cos,
                const float* sin, int64_t row0, int64_t rows, int T, int H, int Hkv, int hd,
                hipStream_t s);
hipError_t swiglu_fwd(int out_dtype, const float* gu, void* act, int64_t M, int F, hipStream_t s);
hipError_t swiglu_bwd(int out_dtype, const float* gu, const float* dact, void* dgu, int64_t M,
                      int F, hipStream_t s);
hipError_t xent(int out_dtype, const float* logits, const int32_t* targets, float* loss,
                void* dlogits, int64_t rows, int V, float scale, hipStream_t s);
hipError_t cast(int out_dtype, const float* x, void* y, int64_t n, hipStream_t s);

}  // namespace mt
