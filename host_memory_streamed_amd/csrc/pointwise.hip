// Memory-bound kernels of the layer template: RMSNorm forward/backward,
// rotary embedding, SwiGLU, cross-entropy and fp32 -> bf16 casts. Each reads
// and writes its operands once, with 16-byte accesses along rows where the
// row length allows; reductions are wave64 shuffles plus one LDS step, in a
// fixed order so every result is deterministic.
#include "dev_common.h"
#include "kernels.h"

namespace mt {
namespace {

constexpr int RMS_MAX_D = 16384;
constexpr int RMS_BWD_MAX_PARTIALS = 1024;   // four row groups per CU

template <typename T>
__device__ __forceinline__ void store4(T* p, floatx4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, floatx4 v) {
  *reinterpret_cast<floatx4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, floatx4 v) {
  bf16x4 b;
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = to_bf16(v[i]);
  *reinterpret_cast<bf16x4*>(p) = b;
}

// Sum over the 256 threads of a block; every thread gets the result.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// ---------------------------------------------------------------- RMSNorm ---

// One wave per row; d % 4 == 0.
template <typename OutT>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ w,
                                                          OutT* __restrict__ y,
                                                          float* __restrict__ rstd, int64_t rows,
                                                          int d, float eps) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const float* xr = x + row * d;
  float ss = 0.f;
  for (int c = lane * 4; c < d; c += 256) {
    const floatx4 v = *reinterpret_cast<const floatx4*>(xr + c);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / (float)d + eps);
  if (lane == 0) rstd[row] = r;
  OutT* yr = y + row * d;
  for (int c = lane * 4; c < d; c += 256) {
    const floatx4 v = *reinterpret_cast<const floatx4*>(xr + c);
    const floatx4 g = *reinterpret_cast<const floatx4*>(w + c);
    store4<OutT>(yr + c, v * r * g);
  }
}

// Rows [blk*rpb, (blk+1)*rpb) per block; each thread owns columns
// tid*4 + j*1024. dx = r (gw - x r^2 mean(gw x)), gw = dy w; the block's
// partial dw (sum of dy x r over its rows, in row order) goes to ws[blk].
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ w,
                                                          const float* __restrict__ rstd,
                                                          const float* __restrict__ dy, float* dx,
                                                          int accumulate, float* __restrict__ ws,
                                                          int64_t rows, int d, int64_t rpb) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  constexpr int MAXJ = RMS_MAX_D / 1024;
  floatx4 dwp[MAXJ];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) dwp[j] = floatx4{0, 0, 0, 0};
  const int64_t r0 = (int64_t)blockIdx.x * rpb, r1 = min(rows, r0 + rpb);
  for (int64_t row = r0; row < r1; ++row) {
    const float* xr = x + row * d;
    const float* gr = dy + row * d;
    const float r = rstd[row];
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      const int c = tid * 4 + j * 1024;
      if (c < d) {
        const floatx4 xv = *reinterpret_cast<const floatx4*>(xr + c);
        const floatx4 gv = *reinterpret_cast<const floatx4*>(gr + c);
        const floatx4 wv = *reinterpret_cast<const floatx4*>(w + c);
        const floatx4 gw = gv * wv;
        dot += gw[0] * xv[0] + gw[1] * xv[1] + gw[2] * xv[2] + gw[3] * xv[3];
        dwp[j] += gv * xv * r;
      }
    }
    const float mean = block_sum(dot, red) / (float)d;
    const float k = r * r * mean;
    float* dr = dx + row * d;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      const int c = tid * 4 + j * 1024;
      if (c < d) {
        const floatx4 xv = *reinterpret_cast<const floatx4*>(xr + c);
        const floatx4 gv = *reinterpret_cast<const floatx4*>(gr + c);
        const floatx4 wv = *reinterpret_cast<const floatx4*>(w + c);
        floatx4 out = (gv * wv - xv * k) * r;
        if (accumulate) out += *reinterpret_cast<const floatx4*>(dr + c);
        *reinterpret_cast<floatx4*>(dr + c) = out;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int c = tid * 4 + j * 1024;
    if (c < d) *reinterpret_cast<floatx4*>(ws + (int64_t)blockIdx.x * d + c) = dwp[j];
  }
}

// dw[c] = sum over partial rows in order.
// dw[c] = sum over the partial rows, in a fixed order: a block owns 64
// columns (16 float4 groups); its 16 lanes per group sum the partials
// p = lane, lane + 16, ... in order, and the 16 lane sums are added in lane
// order. Reads are 256-byte coalesced rows; d % 4 == 0.
__global__ __launch_bounds__(256) void reduce_rows_kernel(const float* __restrict__ ws, float* __restrict__ dw,
                                                          int nparts, int d, int acc) {
  __shared__ floatx4 part[16][16];
  const int cg = threadIdx.x & 15, pl = threadIdx.x >> 4;
  const int c = blockIdx.x * 64 + cg * 4;
  floatx4 s = floatx4{0.f, 0.f, 0.f, 0.f};
  if (c < d)
    for (int p = pl; p < nparts; p += 16) s += *reinterpret_cast<const floatx4*>(ws + (int64_t)p * d + c);
  part[pl][cg] = s;
  __syncthreads();
  if (pl == 0 && c < d) {
    floatx4 t = part[0][cg];
#pragma unroll
    for (int q = 1; q < 16; ++q) t += part[q][cg];
#pragma unroll
    for (int e = 0; e < 4; ++e) dw[c + e] = acc ? dw[c + e] + t[e] : t[e];   // dw needs no alignment
  }
}

// ------------------------------------------------------------------- RoPE ---

// One block per token; columns of the packed [q heads | k heads | v heads] row.
template <typename OutT>
__global__ __launch_bounds__(256) void rope_kernel(const float* __restrict__ in, OutT* __restrict__ out,
                                                   const float* __restrict__ cosv,
                                                   const float* __restrict__ sinv, int64_t row0,
                                                   int Tn, int H, int Hkv, int hd, int backward) {
  const int64_t m = blockIdx.x;
  const int t = (int)((row0 + m) % Tn);
  const int half = hd / 2;
  const int rot = (H + Hkv) * half;       // rotated pairs
  const int width = (H + 2 * Hkv) * hd;
  const float* ir = in + m * width;
  OutT* orow = out + m * width;
  const float* cr = cosv + (int64_t)t * half;
  const float* sr = sinv + (int64_t)t * half;
  const int total = rot + Hkv * hd;
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    if (idx < rot) {
      const int head = idx / half, i = idx % half;
      const int c1 = head * hd + i, c2 = c1 + half;
      const float x1 = ir[c1], x2 = ir[c2], cs = cr[i], sn = sr[i];
      float o1, o2;
      if (backward) { o1 = x1 * cs + x2 * sn; o2 = x2 * cs - x1 * sn; }
      else          { o1 = x1 * cs - x2 * sn; o2 = x2 * cs + x1 * sn; }
      orow[c1] = from_f32<OutT>(o1);
      orow[c2] = from_f32<OutT>(o2);
    } else {
      const int c = (H + Hkv) * hd + (idx - rot);
      orow[c] = from_f32<OutT>(ir[c]);
    }
  }
}

// The same rotation four pairs per thread with 16-byte loads (hd % 8 == 0,
// rows and tables 16-byte aligned).
template <typename OutT>
__global__ __launch_bounds__(256) void rope4_kernel(const float* __restrict__ in, OutT* __restrict__ out,
                                                    const float* __restrict__ cosv,
                                                    const float* __restrict__ sinv, int64_t row0,
                                                    int Tn, int H, int Hkv, int hd, int backward) {
  const int64_t m = blockIdx.x;
  const int t = (int)((row0 + m) % Tn);
  const int half = hd / 2, q4 = half / 4;
  const int rot = (H + Hkv) * q4;         // rotated quads
  const int width = (H + 2 * Hkv) * hd;
  const float* ir = in + m * width;
  OutT* orow = out + m * width;
  const float* cr = cosv + (int64_t)t * half;
  const float* sr = sinv + (int64_t)t * half;
  const int total = rot + Hkv * hd / 4;
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    if (idx < rot) {
      const int head = idx / q4, i = (idx % q4) * 4;
      const int c1 = head * hd + i, c2 = c1 + half;
      const floatx4 x1 = *reinterpret_cast<const floatx4*>(ir + c1);
      const floatx4 x2 = *reinterpret_cast<const floatx4*>(ir + c2);
      const floatx4 cs = *reinterpret_cast<const floatx4*>(cr + i);
      const floatx4 sn = *reinterpret_cast<const floatx4*>(sr + i);
      floatx4 o1, o2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (backward) { o1[e] = x1[e] * cs[e] + x2[e] * sn[e]; o2[e] = x2[e] * cs[e] - x1[e] * sn[e]; }
        else          { o1[e] = x1[e] * cs[e] - x2[e] * sn[e]; o2[e] = x2[e] * cs[e] + x1[e] * sn[e]; }
      }
      store4<OutT>(orow + c1, o1);
      store4<OutT>(orow + c2, o2);
    } else {
      const int c = (H + Hkv) * hd + (idx - rot) * 4;
      store4<OutT>(orow + c, *reinterpret_cast<const floatx4*>(ir + c));
    }
  }
}

// ----------------------------------------------------------------- SwiGLU ---

__device__ __forceinline__ float sigmoidf(float x) { return 1.f / (1.f + expf(-x)); }

template <typename OutT>
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const float* __restrict__ gu,
                                                         OutT* __restrict__ act, int64_t M, int F) {
  const int64_t n = M * F;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / F;
    const int f = (int)(i % F);
    const float g = gu[m * 2 * F + f], u = gu[m * 2 * F + F + f];
    act[i] = from_f32<OutT>(g * sigmoidf(g) * u);
  }
}

template <typename OutT>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ gu,
                                                         const float* __restrict__ dact,
                                                         OutT* __restrict__ dgu, int64_t M, int F) {
  const int64_t n = M * F;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / F;
    const int f = (int)(i % F);
    const float g = gu[m * 2 * F + f], u = gu[m * 2 * F + F + f], da = dact[i];
    const float s = sigmoidf(g);
    dgu[m * 2 * F + f] = from_f32<OutT>(da * u * s * (1.f + g * (1.f - s)));
    dgu[m * 2 * F + F + f] = from_f32<OutT>(da * g * s);
  }
}

// Four consecutive f per thread (F % 4 == 0, 16-byte aligned gu and dact,
// act / dgu aligned to four elements): one row per blockIdx.y step, 16-byte
// loads, no per-element index division. Same arithmetic per element as the
// kernels above.
template <typename OutT>
__global__ __launch_bounds__(256) void swiglu_fwd4_kernel(const float* __restrict__ gu,
                                                          OutT* __restrict__ act, int64_t M, int F) {
  const int F4 = F / 4;
  for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
    const floatx4* g4 = reinterpret_cast<const floatx4*>(gu + m * 2 * F);
    const floatx4* u4 = reinterpret_cast<const floatx4*>(gu + m * 2 * F + F);
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < F4; j += gridDim.x * blockDim.x) {
      const floatx4 g = g4[j], u = u4[j];
      floatx4 a;
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = g[e] * sigmoidf(g[e]) * u[e];
      store4<OutT>(act + m * F + 4 * j, a);
    }
  }
}

template <typename OutT>
__global__ __launch_bounds__(256) void swiglu_bwd4_kernel(const float* __restrict__ gu,
                                                          const float* __restrict__ dact,
                                                          OutT* __restrict__ dgu, int64_t M, int F) {
  const int F4 = F / 4;
  for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
    const floatx4* g4 = reinterpret_cast<const floatx4*>(gu + m * 2 * F);
    const floatx4* u4 = reinterpret_cast<const floatx4*>(gu + m * 2 * F + F);
    const floatx4* d4 = reinterpret_cast<const floatx4*>(dact + m * F);
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < F4; j += gridDim.x * blockDim.x) {
      const floatx4 g = g4[j], u = u4[j], da = d4[j];
      floatx4 dg, du;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sg = sigmoidf(g[e]);
        dg[e] = da[e] * u[e] * sg * (1.f + g[e] * (1.f - sg));
        du[e] = da[e] * g[e] * sg;
      }
      store4<OutT>(dgu + m * 2 * F + 4 * j, dg);
      store4<OutT>(dgu + m * 2 * F + F + 4 * j, du);
    }
  }
}

// grid of the row-wise vector kernels: blocks across a row's F/4 groups,
// rows strided over at most 8192 block rows
dim3 grid4(int64_t M, int F) {
  const int bx = (F / 4 + 255) / 256;
  return dim3((unsigned)bx, (unsigned)(M < 8192 ? M : 8192));
}

bool vec4_ok(int F, const void* a, const void* b, const void* c, size_t out_bytes) {
  const uintptr_t o = out_bytes == 2 ? 7 : 15;
  return F % 4 == 0 && (reinterpret_cast<uintptr_t>(a) & 15) == 0 && (reinterpret_cast<uintptr_t>(b) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(c) & o) == 0;
}

// ---------------------------------------------------------- cross-entropy ---

// One block per row: logsumexp by an online max/sum per thread, then
// dlogits = scale * (softmax - onehot).
template <typename OutT>
__global__ __launch_bounds__(256) void xent_kernel(const float* logits, const int32_t* __restrict__ targets,
                                                   float* __restrict__ loss, OutT* dlogits, int V,
                                                   float scale) {
  __shared__ float rm[4], rs[4];
  const int64_t row = blockIdx.x;
  const float* z = logits + row * (int64_t)V;
  float mx = -INFINITY, s = 0.f;
  for (int i = threadIdx.x; i < V; i += 256) {
    const float v = z[i];
    if (v > mx) { s = s * expf(mx - v) + 1.f; mx = v; }
    else s += expf(v - mx);
  }
  // wave then block combine of (max, sum)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(mx, o, WAVE), s2 = __shfl_xor(s, o, WAVE);
    const float mn = fmaxf(mx, m2);
    s = (mx == -INFINITY ? 0.f : s * expf(mx - mn)) + (m2 == -INFINITY ? 0.f : s2 * expf(m2 - mn));
    mx = mn;
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { rm[w] = mx; rs[w] = s; }
  __syncthreads();
  float M4 = fmaxf(fmaxf(rm[0], rm[1]), fmaxf(rm[2], rm[3]));
  float S4 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) S4 += rs[i] * expf(rm[i] - M4);
  const float lse = M4 + logf(S4);
  const int tgt = targets[row];
  // The thread that owns the target element reads it and writes the loss
  // before overwriting it: with dlogits aliasing logits no other thread reads
  // an element that a different thread writes.
  OutT* dz = dlogits + row * (int64_t)V;
  for (int i = threadIdx.x; i < V; i += 256) {
    const float zi = z[i];
    const float p = expf(zi - lse);
    if (i == tgt) loss[row] = lse - zi;
    dz[i] = from_f32<OutT>(scale * (i == tgt ? p - 1.f : p));
  }
}

template <typename OutT>
__global__ void cast_kernel(const float* __restrict__ x, OutT* __restrict__ y, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    y[i] = from_f32<OutT>(x[i]);
}

// Eight elements per thread: two 16-byte loads, one 16-byte store (n8 groups
// of eight; x and y 16-byte aligned).
__global__ void cast8_bf16_kernel(const float* __restrict__ x, bf16* __restrict__ y, int64_t n8) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    const floatx4 a = reinterpret_cast<const floatx4*>(x)[2 * i];
    const floatx4 b = reinterpret_cast<const floatx4*>(x)[2 * i + 1];
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] = to_bf16(a[e]);
      o[4 + e] = to_bf16(b[e]);
    }
    reinterpret_cast<bf16x8*>(y)[i] = o;
  }
}

unsigned grid_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (unsigned)b;
}

}  // namespace

int rmsnorm_bwd_partials(int64_t rows) {
  return (int)(rows < RMS_BWD_MAX_PARTIALS ? (rows < 1 ? 1 : rows) : RMS_BWD_MAX_PARTIALS);
}

hipError_t rmsnorm_fwd(int out_dtype, const float* x, const float* w, void* y, float* rstd,
                       int64_t rows, int d, float eps, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const unsigned g = (unsigned)((rows + 3) / 4);
  if (out_dtype == 1)
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<bf16>, dim3(g), dim3(256), 0, s, x, w, (bf16*)y, rstd, rows, d, eps);
  else
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<float>, dim3(g), dim3(256), 0, s, x, w, (float*)y, rstd, rows, d, eps);
  return hipGetLastError();
}

hipError_t rmsnorm_bwd(const float* x, const float* w, const float* rstd, const float* dy,
                       float* dx, int accumulate, float* dw, float* ws, int64_t rows, int d,
                       hipStream_t s, int dw_accumulate) {
  const int parts = rmsnorm_bwd_partials(rows);
  const int64_t rpb = (rows + parts - 1) / parts;
  if (rows > 0) {
    hipLaunchKernelGGL(rmsnorm_bwd_kernel, dim3(parts), dim3(256), 0, s, x, w, rstd, dy, dx,
                       accumulate, ws, rows, d, rpb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // with no rows the reduction over zero partials writes dw = 0
  const int used = rows > 0 ? (int)((rows + rpb - 1) / rpb) : 0;
  hipLaunchKernelGGL(reduce_rows_kernel, dim3((d + 63) / 64), dim3(256), 0, s, ws, dw, used, d, dw_accumulate);
  return hipGetLastError();
}

hipError_t rope(int out_dtype, int backward, const float* in, void* out, const float* cosv,
                const float* sinv, int64_t row0, int64_t rows, int Tn, int H, int Hkv, int hd,
                hipStream_t s) {
  if (rows == 0) return hipSuccess;
  auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  const bool vec = hd % 8 == 0 && a16(in) && a16(cosv) && a16(sinv) && (out_dtype == 1 ? ((uintptr_t)out & 7) == 0 : a16(out));
  if (vec) {
    if (out_dtype == 1)
      hipLaunchKernelGGL(rope4_kernel<bf16>, dim3((unsigned)rows), dim3(256), 0, s, in, (bf16*)out, cosv, sinv, row0, Tn, H, Hkv, hd, backward);
    else
      hipLaunchKernelGGL(rope4_kernel<float>, dim3((unsigned)rows), dim3(256), 0, s, in, (float*)out, cosv, sinv, row0, Tn, H, Hkv, hd, backward);
  } else if (out_dtype == 1) {
    hipLaunchKernelGGL(rope_kernel<bf16>, dim3((unsigned)rows), dim3(256), 0, s, in, (bf16*)out, cosv, sinv, row0, Tn, H, Hkv, hd, backward);
  } else {
    hipLaunchKernelGGL(rope_kernel<float>, dim3((unsigned)rows), dim3(256), 0, s, in, (float*)out, cosv, sinv, row0, Tn, H, Hkv, hd, backward);
  }
  return hipGetLastError();
}

hipError_t swiglu_fwd(int out_dtype, const float* gu, void* act, int64_t M, int F, hipStream_t s) {
  if (M * F == 0) return hipSuccess;
  if (vec4_ok(F, gu, gu, act, out_dtype == 1 ? 2 : 4)) {
    if (out_dtype == 1)
      hipLaunchKernelGGL(swiglu_fwd4_kernel<bf16>, grid4(M, F), dim3(256), 0, s, gu, (bf16*)act, M, F);
    else
      hipLaunchKernelGGL(swiglu_fwd4_kernel<float>, grid4(M, F), dim3(256), 0, s, gu, (float*)act, M, F);
  } else if (out_dtype == 1) {
    hipLaunchKernelGGL(swiglu_fwd_kernel<bf16>, dim3(grid_for(M * F)), dim3(256), 0, s, gu, (bf16*)act, M, F);
  } else {
    hipLaunchKernelGGL(swiglu_fwd_kernel<float>, dim3(grid_for(M * F)), dim3(256), 0, s, gu, (float*)act, M, F);
  }
  return hipGetLastError();
}

hipError_t swiglu_bwd(int out_dtype, const float* gu, const float* dact, void* dgu, int64_t M, int F,
                      hipStream_t s) {
  if (M * F == 0) return hipSuccess;
  if (vec4_ok(F, gu, dact, dgu, out_dtype == 1 ? 2 : 4)) {
    if (out_dtype == 1)
      hipLaunchKernelGGL(swiglu_bwd4_kernel<bf16>, grid4(M, F), dim3(256), 0, s, gu, dact, (bf16*)dgu, M, F);
    else
      hipLaunchKernelGGL(swiglu_bwd4_kernel<float>, grid4(M, F), dim3(256), 0, s, gu, dact, (float*)dgu, M, F);
  } else if (out_dtype == 1) {
    hipLaunchKernelGGL(swiglu_bwd_kernel<bf16>, dim3(grid_for(M * F)), dim3(256), 0, s, gu, dact, (bf16*)dgu, M, F);
  } else {
    hipLaunchKernelGGL(swiglu_bwd_kernel<float>, dim3(grid_for(M * F)), dim3(256), 0, s, gu, dact, (float*)dgu, M, F);
  }
  return hipGetLastError();
}

hipError_t xent(int out_dtype, const float* logits, const int32_t* targets, float* loss,
                void* dlogits, int64_t rows, int V, float scale, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (out_dtype == 1)
    hipLaunchKernelGGL(xent_kernel<bf16>, dim3((unsigned)rows), dim3(256), 0, s, logits, targets, loss, (bf16*)dlogits, V, scale);
  else
    hipLaunchKernelGGL(xent_kernel<float>, dim3((unsigned)rows), dim3(256), 0, s, logits, targets, loss, (float*)dlogits, V, scale);
  return hipGetLastError();
}

hipError_t cast(int out_dtype, const float* x, void* y, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const bool vec = n % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(y) & 15) == 0;
  if (out_dtype == 1 && vec)
    hipLaunchKernelGGL(cast8_bf16_kernel, dim3(grid_for(n / 8)), dim3(256), 0, s, x, (bf16*)y, n / 8);
  else if (out_dtype == 1)
    hipLaunchKernelGGL(cast_kernel<bf16>, dim3(grid_for(n)), dim3(256), 0, s, x, (bf16*)y, n);
  else
    hipLaunchKernelGGL(cast_kernel<float>, dim3(grid_for(n)), dim3(256), 0, s, x, (float*)y, n);
  return hipGetLastError();
}

}  // namespace mt
