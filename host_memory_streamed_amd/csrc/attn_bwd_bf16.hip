// bf16 causal flash-attention backward on the gfx950 32x32x16 matrix cores.
//
// Same operation and rounding points as the generic backward in
// attention.hip: P is recomputed from the saved logsumexp, D = rowsum(dO O)
// in fp32, dO / P / dS are rounded to bf16 before their products, and the
// gradients come from two deterministic passes (no atomics):
//
//  dK/dV pass: a workgroup owns 128 keys of one kv head (4 waves x 32 keys);
//    the wave's K and V stay in registers as the B operands of
//    S = Q K^T and dP = dO V^T (its keys are the columns); 64-query Q and dO
//    tiles of every query head of the group stream through double-buffered
//    LDS; dV^T += dO^T P and dK^T += Q^T dS take P and dS from the
//    accumulators and dO^T, Q^T through the LDS transpose read.
//  dQ pass: a workgroup owns 128 queries of one head (4 waves x 32); the
//    wave's Q and dO stay in registers as the B operands of S^T = K Q^T and
//    dP^T = V dO^T; 64-key K and V tiles stream through double-buffered LDS;
//    dQ^T += K^T dS^T with K^T through the LDS transpose read.
//
// Both write the gradient rows in the output type, optionally rotated back by
// the RoPE angle of their position (the rotation's backward pairs hd column
// i with i + hd/2, which one lane holds together).
#include "dev_common.h"
#include "kernels.h"

namespace mt {
namespace {

constexpr float B_LOG2E = 1.4426950408889634f;
constexpr int BT = 256;   // threads
constexpr int BW = 128;   // keys (dK/dV) or queries (dQ) per workgroup
constexpr int BS = 64;    // rows per streamed tile

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_b;
typedef uint32_t u32x4_b __attribute__((ext_vector_type(4)));

template <int HD>
struct BCfg {
  static constexpr int P = HD + 8;          // LDS row pitch (elements)
  static constexpr int VPR = HD / 8;        // 16-byte vectors per row
  static constexpr int NV = BS * VPR / BT;  // vectors per thread per tile
  static constexpr int NS = HD / 16;        // 16-wide hd steps
  static constexpr int NH = HD / 32;        // 32-row hd sub-tiles
};

template <int HD>
struct Tile64 {
  u32x4_b v[BCfg<HD>::NV];
  __device__ __forceinline__ void fetch(const bf16* __restrict__ src, int64_t ld, int r0, int Tn, int tid) {
    typedef BCfg<HD> C;
    if (r0 + BS <= Tn) {
#pragma unroll
      for (int j = 0; j < C::NV; ++j) {
        const int u = tid + BT * j;
        const int row = u / C::VPR, col = (u % C::VPR) * 8;
        v[j] = *reinterpret_cast<const u32x4_b*>(src + (int64_t)(r0 + row) * ld + col);
      }
    } else {   // the last tile: rows past the end read as zero
#pragma unroll
      for (int j = 0; j < C::NV; ++j) {
        const int u = tid + BT * j;
        const int row = u / C::VPR, col = (u % C::VPR) * 8;
        const int rr = min(r0 + row, Tn - 1);
        const u32x4_b x = *reinterpret_cast<const u32x4_b*>(src + (int64_t)rr * ld + col);
        v[j] = r0 + row < Tn ? x : u32x4_b{0, 0, 0, 0};
      }
    }
  }
  __device__ __forceinline__ void store(bf16* dst, int tid) const {
    typedef BCfg<HD> C;
#pragma unroll
    for (int j = 0; j < C::NV; ++j) {
      const int u = tid + BT * j;
      const int row = u / C::VPR, col = (u % C::VPR) * 8;
      *reinterpret_cast<u32x4_b*>(dst + row * C::P + col) = v[j];
    }
  }
};

// A operand of a 16-row contraction step read transposed from a row-major
// LDS tile: lane (column col0 + lane%32, slot group G) receives rows
// row0 + 4G + 0..3 and row0 + 8 + 4G + 0..3 of its column, the slot order
// of a 32x32 accumulator's rows.
__device__ __forceinline__ bf16x8 tr_operand(const bf16* tile, int pitch, int row0, int col0, int lane) {
  const int k16 = lane >> 4, i16 = lane & 15, G = lane >> 5;
  const bf16* p = tile + (row0 + 4 * G + (i16 >> 2)) * pitch + col0 + 16 * (k16 & 1) + 4 * (i16 & 3);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_b*)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_b*)(p + 8 * pitch));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <typename OutT>
__device__ __forceinline__ void put4b(OutT* p, floatx4 v) {
  if constexpr (sizeof(OutT) == 4) {
    *reinterpret_cast<floatx4*>(p) = v;
  } else {
    bf16x4 b;
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = to_bf16(v[i]);
    *reinterpret_cast<bf16x4*>(p) = b;
  }
}

// Store one head's gradient row held as 32x32 accumulator columns (lane slot
// group G holds hd = ht*32 + r4*8 + G*4 + e): scaled, optionally rotated back.
template <typename OutT, int HD>
__device__ __forceinline__ void store_acc_row(OutT* row, const floatx16 (&acc)[HD / 32], float scale,
                                              const float* cs, const float* sn, int G) {
  constexpr int NH = HD / 32;
  if (!cs) {
#pragma unroll
    for (int ht = 0; ht < NH; ++ht)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        floatx4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[ht][r4 * 4 + e] * scale;
        put4b<OutT>(row + ht * 32 + r4 * 8 + G * 4, v);
      }
    return;
  }
#pragma unroll
  for (int ht = 0; ht < NH / 2; ++ht)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int c0 = ht * 32 + r4 * 8 + G * 4;
      floatx4 o1, o2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x1 = acc[ht][r4 * 4 + e] * scale, x2 = acc[ht + NH / 2][r4 * 4 + e] * scale;
        const float c = cs[c0 + e], s = sn[c0 + e];
        o1[e] = x1 * c + x2 * s;
        o2[e] = x2 * c - x1 * s;
      }
      put4b<OutT>(row + c0, o1);
      put4b<OutT>(row + HD / 2 + c0, o2);
    }
}

// D[b,h,t] = sum_i dO[m, h*HD+i] O[m, h*HD+i] (fp32); dO rounded to bf16.
template <int HD>
__global__ __launch_bounds__(256) void attn_pre_bf16_kernel(const float* __restrict__ o,
                                                           const float* __restrict__ dout,
                                                           bf16* __restrict__ dcast, float* __restrict__ D,
                                                           int64_t rows, int Tn, int H) {
  const int64_t rid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (m, h) pair
  if (rid >= rows) return;
  const int lane = threadIdx.x & 63;
  const int64_t m = rid / H;
  const int h = (int)(rid % H);
  const int64_t off = m * (int64_t)H * HD + h * HD;
  float acc = 0.f;
  for (int i = lane * 2; i < HD; i += 128) {
    const float d0 = dout[off + i], d1 = dout[off + i + 1];
    acc += d0 * o[off + i] + d1 * o[off + i + 1];
    dcast[off + i] = to_bf16(d0);
    dcast[off + i + 1] = to_bf16(d1);
  }
  acc = wave_sum(acc);
  if (lane == 0) {
    const int64_t b = m / Tn, t = m % Tn;
    D[(b * H + h) * Tn + t] = acc;
  }
}

template <int HD, typename OutT>
__global__ __launch_bounds__(BT, 1) void attn_dkv_bf16_kernel(const bf16* __restrict__ qkv,
                                                             const bf16* __restrict__ dcast,
                                                             const float* __restrict__ lse,
                                                             const float* __restrict__ Dv,
                                                             OutT* __restrict__ dqkv,
                                                             const float* __restrict__ rcos,
                                                             const float* __restrict__ rsin, int Tn,
                                                             int H, int Hkv, int nkb, int xcd_groups) {
  typedef BCfg<HD> C;
  __shared__ __attribute__((aligned(16))) bf16 Qs[2][BS * C::P];
  __shared__ __attribute__((aligned(16))) bf16 Os[2][BS * C::P];
  __shared__ __attribute__((aligned(16))) float Ls[2][BS];
  __shared__ __attribute__((aligned(16))) float Dsh[2][BS];

  const int id = blockIdx.x;
  int kvh, kb;
  if (xcd_groups) {
    const int per = (nkb * Hkv) >> 3;
    const int item = (id & 7) * per + (id >> 3);
    kvh = item / nkb;
    kb = item % nkb;   // low key blocks see the most queries: first
  } else {
    kvh = id % Hkv;
    kb = id / Hkv;
  }
  const int b = blockIdx.z;
  const int grp = H / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, G = lane >> 5;
  const int64_t ld = (int64_t)(H + 2 * Hkv) * HD, ldo = (int64_t)H * HD;
  const bf16* base = qkv + (int64_t)b * Tn * ld;
  const bf16* dbase = dcast + (int64_t)b * Tn * ldo;

  const int kw0 = kb * BW + w * 32;   // the wave's first key
  const int key = kw0 + c;
  bf16x8 kf[C::NS], vf[C::NS];
  {
    const bf16* krow = base + (int64_t)min(key, Tn - 1) * ld + (H + kvh) * HD + G * 8;
    const bf16* vrow = base + (int64_t)min(key, Tn - 1) * ld + (H + Hkv + kvh) * HD + G * 8;
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(krow + s * 16);
      const bf16x8 y = *reinterpret_cast<const bf16x8*>(vrow + s * 16);
      kf[s] = key < Tn ? x : bf16x8{};
      vf[s] = key < Tn ? y : bf16x8{};
    }
  }
  floatx16 dk[C::NH], dv[C::NH];
#pragma unroll
  for (int i = 0; i < C::NH; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[i][r] = dv[i][r] = 0.f;
  const float sl2 = B_LOG2E / sqrtf((float)HD);

  // query tiles at or after the block's first key, for every head of the group
  const int qt0 = (kb * BW) / BS;
  const int nqt = (Tn + BS - 1) / BS - qt0;
  const int n_it = grp * nqt;

  Tile64<HD> qr, orr;
  float lv = 0.f;
  auto fetch = [&](int it) {
    const int h = kvh * grp + it / nqt;
    const int q0 = (qt0 + it % nqt) * BS;
    qr.fetch(base + h * HD, ld, q0, Tn, tid);
    orr.fetch(dbase + h * HD, ldo, q0, Tn, tid);
    if (tid < 2 * BS) {
      const int qi = min(q0 + (tid & (BS - 1)), Tn - 1);
      const int64_t idx = ((int64_t)b * H + h) * Tn + qi;
      lv = tid < BS ? lse[idx] * B_LOG2E : Dv[idx];
    }
  };
  auto stash = [&](int buf) {
    qr.store(Qs[buf], tid);
    orr.store(Os[buf], tid);
    if (tid < BS) Ls[buf][tid] = lv;
    else if (tid < 2 * BS) Dsh[buf][tid - BS] = lv;
  };
  fetch(0);
  stash(0);
  __syncthreads();

  for (int it = 0; it < n_it; ++it) {
    const int buf = it & 1;
    const int q0 = (qt0 + it % nqt) * BS;
    const bool more = it + 1 < n_it;
    if (more) fetch(it + 1);
    const bf16* Qb = Qs[buf];
    const bf16* Ob = Os[buf];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int qs0 = q0 + 32 * u;
      if (qs0 + 31 < kw0) continue;   // every query of the sub-tile precedes the wave's keys
      floatx16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
      const bf16* qrow = Qb + (32 * u + c) * C::P + G * 8;
      const bf16* orow = Ob + (32 * u + c) * C::P + G * 8;
#pragma unroll
      for (int ss = 0; ss < C::NS; ++ss) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(qrow + ss * 16);
        const bf16x8 a2 = *reinterpret_cast<const bf16x8*>(orow + ss * 16);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[ss], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, vf[ss], dp, 0, 0, 0);
      }
      // rows are queries qs0 + (r/4)*8 + G*4 + r%4, the column is this lane's
      // key; masking only where the sub-tile meets the diagonal or the end
      const bool edge = qs0 < kw0 + 31 || qs0 + 31 >= Tn;
      bf16x8 pb0, pb1, db0, db1;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int qr4 = 32 * u + r4 * 8 + G * 4;
        const floatx4 lq = *reinterpret_cast<const floatx4*>(&Ls[buf][qr4]);
        const floatx4 dq4 = *reinterpret_cast<const floatx4*>(&Dsh[buf][qr4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = r4 * 4 + e;
          float pv = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -lq[e]));
          if (edge) {
            const int qi = q0 + qr4 + e;
            if (!(key <= qi && qi < Tn)) pv = 0.f;
          }
          const float dsv = pv * (dp[r] - dq4[e]);
          if (r < 8) { pb0[r] = to_bf16(pv); db0[r] = to_bf16(dsv); }
          else { pb1[r - 8] = to_bf16(pv); db1[r - 8] = to_bf16(dsv); }
        }
      }
#pragma unroll
      for (int ht = 0; ht < C::NH; ++ht) {
        dv[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(Ob, C::P, 32 * u, ht * 32, lane), pb0, dv[ht], 0, 0, 0);
        dv[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(Ob, C::P, 32 * u + 16, ht * 32, lane), pb1, dv[ht], 0, 0, 0);
        dk[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(Qb, C::P, 32 * u, ht * 32, lane), db0, dk[ht], 0, 0, 0);
        dk[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(Qb, C::P, 32 * u + 16, ht * 32, lane), db1, dk[ht], 0, 0, 0);
      }
    }
    if (more) stash(buf ^ 1);
    __syncthreads();
  }

  if (key < Tn) {
    OutT* row = dqkv + ((int64_t)b * Tn + key) * ld;   // dqkv has the qkv layout
    const float* cs = rcos ? rcos + (int64_t)key * (HD / 2) : nullptr;
    const float* sn = rsin ? rsin + (int64_t)key * (HD / 2) : nullptr;
    store_acc_row<OutT, HD>(row + (H + kvh) * HD, dk, 1.f / sqrtf((float)HD), cs, sn, G);
    store_acc_row<OutT, HD>(row + (H + Hkv + kvh) * HD, dv, 1.f, nullptr, nullptr, G);
  }
}

template <int HD, typename OutT>
__global__ __launch_bounds__(BT, 2) void attn_dq_bf16_kernel(const bf16* __restrict__ qkv,
                                                            const bf16* __restrict__ dcast,
                                                            const float* __restrict__ lse,
                                                            const float* __restrict__ Dv,
                                                            OutT* __restrict__ dqkv,
                                                            const float* __restrict__ rcos,
                                                            const float* __restrict__ rsin, int Tn,
                                                            int H, int Hkv, int nq, int xcd_groups) {
  typedef BCfg<HD> C;
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][BS * C::P];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][BS * C::P];

  const int id = blockIdx.x;
  int h, qb;
  if (xcd_groups) {
    const int per = (nq * H) >> 3;
    const int item = (id & 7) * per + (id >> 3);
    h = item / nq;
    qb = nq - 1 - item % nq;
  } else {
    h = id % H;
    qb = nq - 1 - id / H;
  }
  const int b = blockIdx.z;
  const int kvh = h / (H / Hkv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, G = lane >> 5;
  const int64_t ld = (int64_t)(H + 2 * Hkv) * HD, ldo = (int64_t)H * HD;
  const bf16* base = qkv + (int64_t)b * Tn * ld;
  const bf16* Kg = base + (H + kvh) * HD;
  const bf16* Vg = base + (H + Hkv + kvh) * HD;

  const int wq0 = qb * BW + w * 32;
  const int q = wq0 + c;
  const int qc = min(q, Tn - 1);
  bf16x8 qf[C::NS], df[C::NS];
  {
    const bf16* qrow = base + (int64_t)qc * ld + h * HD + G * 8;
    const bf16* drow = dcast + ((int64_t)b * Tn + qc) * ldo + h * HD + G * 8;
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(qrow + s * 16);
      const bf16x8 y = *reinterpret_cast<const bf16x8*>(drow + s * 16);
      qf[s] = q < Tn ? x : bf16x8{};
      df[s] = q < Tn ? y : bf16x8{};
    }
  }
  const int64_t li = ((int64_t)b * H + h) * Tn + qc;
  const float lse2 = q < Tn ? lse[li] * B_LOG2E : 0.f;
  const float Dq = q < Tn ? Dv[li] : 0.f;
  const float sl2 = B_LOG2E / sqrtf((float)HD);
  floatx16 dq[C::NH];
#pragma unroll
  for (int i = 0; i < C::NH; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[i][r] = 0.f;

  const int q_hi = min(Tn, qb * BW + BW);
  const int n_kt = (q_hi - 1) / BS + 1;
  Tile64<HD> kr, vr;
  kr.fetch(Kg, ld, 0, Tn, tid);
  vr.fetch(Vg, ld, 0, Tn, tid);
  kr.store(Ks[0], tid);
  vr.store(Vs[0], tid);
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    const int k0 = kt * BS;
    const bool more = kt + 1 < n_kt;
    if (more) {
      kr.fetch(Kg, ld, k0 + BS, Tn, tid);
      vr.fetch(Vg, ld, k0 + BS, Tn, tid);
    }
    const bf16* Kb = Ks[buf];
    const bf16* Vb = Vs[buf];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int kb0 = k0 + 32 * st;
      if (kb0 > wq0 + 31) continue;   // every key of the sub-tile follows the wave's queries
      floatx16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
      const bf16* krow = Kb + (32 * st + c) * C::P + G * 8;
      const bf16* vrow = Vb + (32 * st + c) * C::P + G * 8;
#pragma unroll
      for (int ss = 0; ss < C::NS; ++ss) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + ss * 16);
        const bf16x8 a2 = *reinterpret_cast<const bf16x8*>(vrow + ss * 16);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ss], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, df[ss], dp, 0, 0, 0);
      }
      // rows are keys kb0 + (r/4)*8 + G*4 + r%4, the column is this lane's
      // query; masking only where the sub-tile meets the diagonal or the end
      const bool edge = kb0 + 31 > wq0 || wq0 + 31 >= Tn;
      bf16x8 db0, db1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -lse2));
        if (edge) {
          const int kk = kb0 + (r >> 2) * 8 + G * 4 + (r & 3);
          if (!(kk <= q && q < Tn)) pv = 0.f;
        }
        const float dsv = pv * (dp[r] - Dq);
        if (r < 8) db0[r] = to_bf16(dsv);
        else db1[r - 8] = to_bf16(dsv);
      }
#pragma unroll
      for (int ht = 0; ht < C::NH; ++ht) {
        dq[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(Kb, C::P, 32 * st, ht * 32, lane), db0, dq[ht], 0, 0, 0);
        dq[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(Kb, C::P, 32 * st + 16, ht * 32, lane), db1, dq[ht], 0, 0, 0);
      }
    }
    if (more) {
      kr.store(Ks[buf ^ 1], tid);
      vr.store(Vs[buf ^ 1], tid);
    }
    __syncthreads();
  }

  if (q < Tn) {
    OutT* row = dqkv + ((int64_t)b * Tn + q) * ld + h * HD;
    const float* cs = rcos ? rcos + (int64_t)q * (HD / 2) : nullptr;
    const float* sn = rsin ? rsin + (int64_t)q * (HD / 2) : nullptr;
    store_acc_row<OutT, HD>(row, dq, 1.f / sqrtf((float)HD), cs, sn, G);
  }
}

template <int HD, typename OutT>
hipError_t launch_bwd(const void* qkv, const float* o, const float* dout, const float* lse, void* dqkv,
                      const float* rcos, const float* rsin, void* ws, int B, int Tn, int H, int Hkv,
                      hipStream_t s) {
  const int64_t M = (int64_t)B * Tn;
  float* D = reinterpret_cast<float*>(ws);
  bf16* dcast = reinterpret_cast<bf16*>(reinterpret_cast<char*>(ws) + attn_ws_d_bytes(B, Tn, H));
  const int64_t rows = M * H;
  hipLaunchKernelGGL((attn_pre_bf16_kernel<HD>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, o, dout,
                     dcast, D, rows, Tn, H);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb = (Tn + BW - 1) / BW;
  const int64_t kv_items = (int64_t)nb * Hkv, q_items = (int64_t)nb * H;
  hipLaunchKernelGGL((attn_dkv_bf16_kernel<HD, OutT>), dim3((unsigned)kv_items, 1, B), dim3(BT), 0, s,
                     (const bf16*)qkv, (const bf16*)dcast, lse, (const float*)D, (OutT*)dqkv, rcos, rsin,
                     Tn, H, Hkv, nb, (int)((kv_items % 8 == 0) && (Hkv % 8 == 0)));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_dq_bf16_kernel<HD, OutT>), dim3((unsigned)q_items, 1, B), dim3(BT), 0, s,
                     (const bf16*)qkv, (const bf16*)dcast, lse, (const float*)D, (OutT*)dqkv, rcos, rsin,
                     Tn, H, Hkv, nb, (int)((q_items % 8 == 0) && (H % 8 == 0)));
  return hipGetLastError();
}

}  // namespace

hipError_t attn_bwd_bf16(const void* qkv, const float* o, const float* dout, const float* lse, void* dqkv,
                         int out_dtype, const float* rcos, const float* rsin, void* ws, int B, int Tn,
                         int H, int Hkv, int hd, hipStream_t s) {
  if (hd == 64)
    return out_dtype ? launch_bwd<64, bf16>(qkv, o, dout, lse, dqkv, rcos, rsin, ws, B, Tn, H, Hkv, s)
                     : launch_bwd<64, float>(qkv, o, dout, lse, dqkv, rcos, rsin, ws, B, Tn, H, Hkv, s);
  return out_dtype ? launch_bwd<128, bf16>(qkv, o, dout, lse, dqkv, rcos, rsin, ws, B, Tn, H, Hkv, s)
                   : launch_bwd<128, float>(qkv, o, dout, lse, dqkv, rcos, rsin, ws, B, Tn, H, Hkv, s);
}

}  // namespace mt
