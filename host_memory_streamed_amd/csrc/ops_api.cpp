// C ABI of the individual kernels (mt_ops.h): host-side argument checks, then
// one launch on the caller's stream.
#include "kernels.h"
#include "runtime.h"

using namespace mt;

namespace {

int hip_rc(hipError_t e) { return e == hipSuccess ? MT_OK : MT_EHIP; }
bool dtype_ok(int32_t t) { return t == MT_FP32 || t == MT_BF16; }
hipStream_t st(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int mt_op_gemm(int32_t dtype, int32_t layout, const void* A, int64_t lda, const void* B, int64_t ldb,
               float* C, int64_t ldc, const float* R, int64_t ldr, int64_t M, int64_t N, int64_t K,
               void* stream) {
  return mt_op_gemm_variant(dtype, layout, A, lda, B, ldb, C, ldc, R, ldr, M, N, K, 0, stream);
}

int mt_op_gemm_variant(int32_t dtype, int32_t layout, const void* A, int64_t lda, const void* B,
                       int64_t ldb, float* C, int64_t ldc, const float* R, int64_t ldr, int64_t M,
                       int64_t N, int64_t K, int32_t variant, void* stream) {
  if (variant < 0 || variant > 2) return MT_EINVAL;
  if (!dtype_ok(dtype) || layout < MT_GEMM_NT || layout > MT_GEMM_TN) return MT_EINVAL;
  if (M < 0 || N < 0 || K < 0 || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return MT_EINVAL;
  if (M == 0 || N == 0) return MT_OK;
  if (!C || (K > 0 && (!A || !B))) return MT_EINVAL;
  // leading dimensions as stored: NT A[M][lda] B[N][ldb]; NN A[M][lda] B[K][ldb]; TN A[K][lda] B[K][ldb]
  const int64_t a_cols = layout == MT_GEMM_TN ? M : K;
  const int64_t b_cols = layout == MT_GEMM_NT ? K : N;
  if (lda < a_cols || ldb < b_cols || ldc < N || (R && ldr < N)) return MT_EINVAL;
  return hip_rc(gemm_variant(dtype, layout, A, lda, B, ldb, C, ldc, R, ldr, M, N, K, variant, st(stream)));
}

int64_t mt_op_gemm_ws_bytes(void) { return GEMM_WS_BYTES; }

int mt_op_gemm_ws(int32_t dtype, int32_t layout, const void* A, int64_t lda, const void* B, int64_t ldb,
                  float* C, int64_t ldc, const float* R, int64_t ldr, int64_t M, int64_t N, int64_t K,
                  void* ws, int64_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype) || layout < MT_GEMM_NT || layout > MT_GEMM_TN) return MT_EINVAL;
  if (M < 0 || N < 0 || K < 0 || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX || ws_bytes < 0) return MT_EINVAL;
  if (ws_bytes > 0 && (!ws || ((uintptr_t)ws & 15))) return MT_EINVAL;
  if (M == 0 || N == 0) return MT_OK;
  if (!C || (K > 0 && (!A || !B))) return MT_EINVAL;
  const int64_t a_cols = layout == MT_GEMM_TN ? M : K;
  const int64_t b_cols = layout == MT_GEMM_NT ? K : N;
  if (lda < a_cols || ldb < b_cols || ldc < N || (R && ldr < N)) return MT_EINVAL;
  return hip_rc(gemm_ws(dtype, layout, A, lda, B, ldb, C, ldc, R, ldr, M, N, K, ws_bytes > 0 ? ws : nullptr,
                        ws_bytes, st(stream)));
}

int mt_op_rmsnorm_fwd(int32_t out_dtype, const float* x, const float* w, void* y, float* rstd, int64_t rows,
                      int32_t d, float eps, void* stream) {
  if (!dtype_ok(out_dtype) || rows < 0 || d < 4 || d % 4 || d > 16384) return MT_EINVAL;
  if (rows == 0) return MT_OK;
  if (!x || !w || !y || !rstd) return MT_EINVAL;
  return hip_rc(rmsnorm_fwd(out_dtype, x, w, y, rstd, rows, d, eps, st(stream)));
}

int64_t mt_op_rmsnorm_bwd_ws_floats(int64_t rows, int32_t d) {
  return (int64_t)rmsnorm_bwd_partials(rows) * d;
}

int mt_op_rmsnorm_bwd(const float* x, const float* w, const float* rstd, const float* dy, float* dx,
                      int32_t accumulate, float* dw, float* ws, int64_t rows, int32_t d, void* stream) {
  if (rows < 0 || d < 4 || d % 4 || d > 16384 || !w || !dw || !ws) return MT_EINVAL;
  if (rows > 0 && (!x || !rstd || !dy || !dx)) return MT_EINVAL;
  auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (!a16(w) || !a16(ws) || (rows > 0 && (!a16(x) || !a16(dy) || !a16(dx)))) return MT_EINVAL;
  return hip_rc(rmsnorm_bwd(x, w, rstd, dy, dx, accumulate, dw, ws, rows, d, st(stream)));
}

static int rope_check(int32_t out_dtype, const void* in, void* out, const float* c, const float* s, int32_t B,
                      int32_t T, int32_t H, int32_t Hkv, int32_t hd) {
  if (!dtype_ok(out_dtype) || B < 0 || T < 0 || H < 1 || Hkv < 1 || hd < 2 || hd % 2) return MT_EINVAL;
  if ((int64_t)B * T >= MAX_BLOCK_ROWS) return MT_EINVAL;   // one block per token row
  if ((int64_t)B * T > 0 && (!in || !out || !c || !s)) return MT_EINVAL;
  return MT_OK;
}

int mt_op_rope_fwd(int32_t out_dtype, const float* qkv, void* out, const float* cos, const float* sin,
                   int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t hd, void* stream) {
  int rc = rope_check(out_dtype, qkv, out, cos, sin, B, T, H, Hkv, hd);
  if (rc) return rc;
  return hip_rc(rope(out_dtype, 0, qkv, out, cos, sin, 0, (int64_t)B * T, T, H, Hkv, hd, st(stream)));
}

int mt_op_rope_bwd(int32_t out_dtype, const float* dqkv, void* out, const float* cos, const float* sin,
                   int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t hd, void* stream) {
  int rc = rope_check(out_dtype, dqkv, out, cos, sin, B, T, H, Hkv, hd);
  if (rc) return rc;
  return hip_rc(rope(out_dtype, 1, dqkv, out, cos, sin, 0, (int64_t)B * T, T, H, Hkv, hd, st(stream)));
}

static int attn_check(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t hd) {
  if (!dtype_ok(dtype) || !attn_supported(dtype, hd)) return MT_EINVAL;
  if (B < 0 || T < 0 || H < 1 || Hkv < 1 || H % Hkv) return MT_EINVAL;
  if (B > 65535 || H > 65535) return MT_EINVAL;
  // tile byte offsets of the direct copies, and work-items per grid dimension
  // (one 256-thread workgroup per 64 queries or keys and head, at most)
  if ((int64_t)(H + 2 * Hkv) * hd >= MAX_ATTN_LD) return MT_EINVAL;
  if (((int64_t)T + 63) / 64 * H * 256 >= (1ll << 32)) return MT_EINVAL;
  return MT_OK;
}

int mt_op_attn_fwd(int32_t dtype, const void* qkv, float* o, void* o_cast, float* lse, int32_t B, int32_t T,
                   int32_t H, int32_t Hkv, int32_t hd, void* stream) {
  int rc = attn_check(dtype, B, T, H, Hkv, hd);
  if (rc) return rc;
  if ((int64_t)B * T == 0) return MT_OK;
  if (!qkv || !o || !lse) return MT_EINVAL;
  return hip_rc(attn_fwd(dtype, qkv, o, o_cast, lse, B, T, H, Hkv, hd, st(stream)));
}

int64_t mt_op_attn_bwd_ws_bytes(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t hd) {
  return attn_ws_d_bytes(B, T, H) + (int64_t)B * T * H * hd * (dtype == MT_BF16 ? 2 : 4) +
         (dtype == MT_BF16 ? attn_dkv_part_bytes(B, T, H, hd) : 0);
}

int mt_op_attn_bwd(int32_t dtype, const void* qkv, const float* o, const float* dout, const float* lse,
                   float* dqkv, void* ws, int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t hd,
                   void* stream) {
  int rc = attn_check(dtype, B, T, H, Hkv, hd);
  if (rc) return rc;
  if ((int64_t)B * T == 0) return MT_OK;
  if (!qkv || !o || !dout || !lse || !dqkv || !ws) return MT_EINVAL;
  return hip_rc(attn_bwd(dtype, qkv, o, dout, lse, dqkv, MT_FP32, nullptr, nullptr, ws, B, T, H, Hkv, hd,
                         st(stream)));
}

int mt_op_attn_bwd_rope(int32_t dtype, const void* qkv, const float* o, const float* dout, const float* lse,
                        const float* cos, const float* sin, void* dqkv, void* ws, int32_t B, int32_t T,
                        int32_t H, int32_t Hkv, int32_t hd, void* stream) {
  int rc = attn_check(dtype, B, T, H, Hkv, hd);
  if (rc) return rc;
  if ((int64_t)B * T == 0) return MT_OK;
  if (!qkv || !o || !dout || !lse || !cos || !sin || !dqkv || !ws) return MT_EINVAL;
  return hip_rc(attn_bwd(dtype, qkv, o, dout, lse, dqkv, dtype, cos, sin, ws, B, T, H, Hkv, hd, st(stream)));
}

int mt_op_swiglu_fwd(int32_t out_dtype, const float* gu, void* act, int64_t M, int32_t F, void* stream) {
  if (!dtype_ok(out_dtype) || M < 0 || F < 1) return MT_EINVAL;
  if (M == 0) return MT_OK;
  if (!gu || !act) return MT_EINVAL;
  return hip_rc(swiglu_fwd(out_dtype, gu, act, M, F, st(stream)));
}

int mt_op_swiglu_bwd(int32_t out_dtype, const float* gu, const float* dact, void* dgu, int64_t M, int32_t F,
                     void* stream) {
  if (!dtype_ok(out_dtype) || M < 0 || F < 1) return MT_EINVAL;
  if (M == 0) return MT_OK;
  if (!gu || !dact || !dgu) return MT_EINVAL;
  return hip_rc(swiglu_bwd(out_dtype, gu, dact, dgu, M, F, st(stream)));
}

int mt_op_xent(int32_t out_dtype, const float* logits, const int32_t* targets, float* loss, void* dlogits,
               int64_t rows, int32_t V, float scale, void* stream) {
  if (!dtype_ok(out_dtype) || rows < 0 || rows >= MAX_BLOCK_ROWS || V < 1) return MT_EINVAL;
  if (rows == 0) return MT_OK;
  if (!logits || !targets || !loss || !dlogits) return MT_EINVAL;
  return hip_rc(xent(out_dtype, logits, targets, loss, dlogits, rows, V, scale, st(stream)));
}

int mt_op_cast(int32_t out_dtype, const float* x, void* y, int64_t n, void* stream) {
  if (!dtype_ok(out_dtype) || n < 0) return MT_EINVAL;
  if (n == 0) return MT_OK;
  if (!x || !y) return MT_EINVAL;
  return hip_rc(cast(out_dtype, x, y, n, st(stream)));
}

}  // extern "C"
