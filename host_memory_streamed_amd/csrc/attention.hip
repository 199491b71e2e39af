// Causal grouped-query flash attention on the gfx950 matrix cores.
//
// Inputs are the packed, rotated projections qkv [M, (H + 2 Hkv) hd] (q heads,
// k heads, v heads per token; M = B*T in (b, t) order) in fp32 or bf16. Query
// head h reads kv head h / (H/Hkv); scale 1/sqrt(hd); key j is visible to
// query i iff j <= i.
//
// Matrix-core usage (16x16 family, see dev_common.h): every product is laid
// out so that its B operand is either a row fragment held in registers or the
// fp32 accumulator of the previous product, which removes any register
// shuffles between products:
//   forward / dQ pass : S^T = K Q^T  (keys are rows, the lane's query is the
//                       column), O^T += V^T P^T, dP^T = V dO^T,
//                       dQ^T += K^T dS^T;
//   dK/dV pass        : S = Q K^T (the lane's key is the column),
//                       dV^T += dO^T P, dK^T += Q^T dS.
// A row fragment puts hd range [g*hd/4, (g+1)*hd/4) in lane group g = lane/16.
// When an accumulator (rows c = t*16 + g*4 + r) feeds the next product as its
// B operand, the contraction runs over those rows in the same slot order on
// both operands, so the A operand needs 4 consecutive contraction entries per
// 16-row sub-tile: bf16 gets them from the row-major tile with the LDS
// transpose read (ds_read_b64_tr_b16); fp32 reads an explicitly transposed
// LDS copy.
//
// Online softmax keeps a running max and sum per query in the log2 domain.
// In bf16 mode P (for P.V and for dV) and dS are rounded to bf16 before their
// products; D = rowsum(dO * O) uses fp32 dO and O. The backward recomputes P
// from the saved logsumexp and runs two passes (dK/dV over key blocks, dQ over
// query blocks) so that no accumulation races.
#include "dev_common.h"
#include "kernels.h"

namespace mt {
namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

template <typename T, int HD>
struct Cfg {
  typedef Mfma16<T> MF;
  static constexpr int KL = MF::KL;
  static constexpr int HQ = HD / 4;              // row-fragment length per lane
  static constexpr int NSH = HQ / KL;            // instructions for a contraction over hd
  static constexpr int HT = HD / 16;             // 16-row tiles over hd
  static constexpr int VE = 16 / sizeof(T);      // elements per 16-byte vector
  static constexpr int PAD = VE;                 // LDS row padding (elements)
  static constexpr int BKV = sizeof(T) == 2 ? 64 : 32;  // keys per tile (forward, dQ)
  static constexpr int BQ = sizeof(T) == 2 ? 64 : 16;   // queries per tile (dK/dV)
  // bf16 reads transposed operands straight from the row-major tiles with the
  // LDS transpose read; fp32 keeps explicitly transposed copies
  static constexpr bool TR = sizeof(T) == 2;
};

// Copy n_rows rows of HD elements (global row stride ld, rows >= valid are
// zero) into an LDS tile [row][HD + PAD].
template <typename T, int HD>
__device__ __forceinline__ void load_rows(T* dst, const T* __restrict__ src, int64_t ld, int row0,
                                          int n_rows, int valid, int tid) {
  constexpr int VE = Cfg<T, HD>::VE, P = HD + Cfg<T, HD>::PAD;
  constexpr int CPR = HD / VE;
  for (int c = tid; c < n_rows * CPR; c += 256) {
    const int r = c / CPR, col = (c % CPR) * VE;
    Vec16 v = {};
    if (row0 + r < valid) v = *reinterpret_cast<const Vec16*>(src + (int64_t)(row0 + r) * ld + col);
    *reinterpret_cast<Vec16*>(dst + r * P + col) = v;
  }
}

// Same rows written transposed: dst[hd][row], row pitch n_rows + PAD.
template <typename T, int HD>
__device__ __forceinline__ void load_rows_t(T* dst, const T* __restrict__ src, int64_t ld, int row0,
                                            int n_rows, int valid, int tid) {
  constexpr int VE = Cfg<T, HD>::VE;
  constexpr int CPR = HD / VE;
  const int P = n_rows + Cfg<T, HD>::PAD;
  for (int c = tid; c < (n_rows / 2) * CPR; c += 256) {
    const int rp = (c / CPR) * 2, col = (c % CPR) * VE;
    Vec16 a = {}, b = {};
    if (row0 + rp < valid) a = *reinterpret_cast<const Vec16*>(src + (int64_t)(row0 + rp) * ld + col);
    if (row0 + rp + 1 < valid) b = *reinterpret_cast<const Vec16*>(src + (int64_t)(row0 + rp + 1) * ld + col);
    const T* ea = reinterpret_cast<const T*>(&a);
    const T* eb = reinterpret_cast<const T*>(&b);
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      T pair[2] = {ea[e], eb[e]};
      T* d = dst + (col + e) * P + rp;
      if (sizeof(T) == 2) {
        uint32_t u;
        __builtin_memcpy(&u, pair, 4);
        *reinterpret_cast<uint32_t*>(d) = u;
      } else {
        uint2 u;
        __builtin_memcpy(&u, pair, 8);
        *reinterpret_cast<uint2*>(d) = u;
      }
    }
  }
}

// Row fragment from global memory: HQ elements at hd offset g*HQ of row `row`.
template <typename T, int HD, int N>
__device__ __forceinline__ void load_frag(T (&f)[N], const T* __restrict__ src, int64_t ld, int row,
                                          int valid, int g) {
  constexpr int HQ = Cfg<T, HD>::HQ, VE = Cfg<T, HD>::VE;
  static_assert(N == HQ, "fragment length");
#pragma unroll
  for (int i = 0; i < HQ / VE; ++i) {
    Vec16 v = {};
    if (row < valid) v = *reinterpret_cast<const Vec16*>(src + (int64_t)row * ld + g * HQ + i * VE);
    __builtin_memcpy(&f[i * VE], &v, 16);
  }
}

// acc += A_row . B over hd: A from an LDS row (hd offset g*HQ), B from registers.
template <typename T, int HD, int N>
__device__ __forceinline__ floatx4 contract_hd(const T* arow, const T (&b)[N], floatx4 acc) {
  typedef Cfg<T, HD> C;
  static_assert(N == C::HQ, "fragment length");
  typedef typename C::MF MF;
#pragma unroll
  for (int s = 0; s < C::NSH; ++s) {
    typename MF::frag fa = *reinterpret_cast<const typename MF::frag*>(arow + s * C::KL);
    typename MF::frag fb;
    __builtin_memcpy(&fb, &b[s * C::KL], sizeof(fb));
    acc = MF::mma(fa, fb, acc);
  }
  return acc;
}

// B operand built from an fp32 accumulator spanning NT16 16-row sub-tiles.
template <typename T, int NT16>
struct AccFrag;
template <int NT16>
struct AccFrag<bf16, NT16> {
  bf16x8 f[NT16 / 2];
  __device__ __forceinline__ void set(const floatx4 (&p)[NT16]) {
#pragma unroll
    for (int s = 0; s < NT16 / 2; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f[s][r] = to_bf16(p[2 * s][r]);
        f[s][4 + r] = to_bf16(p[2 * s + 1][r]);
      }
  }
  // acc += A . B where A[row][c] = tile[c][col0 + row] of a row-major LDS tile
  // (pitch elements per row): the LDS transpose read gives lane l (group
  // g = l/16, i = l%16) rows row0 + 4g + e, e = 0..3, of column col0 + i when
  // lane 4e + q of the group supplies the address of row row0 + 4g + e,
  // column col0 + 4q. Two reads per slice cover contraction rows
  // 32s + 4g + r and 32s + 16 + 4g + r, the accumulator's slot order.
  __device__ __forceinline__ floatx4 apply_tr(const bf16* tile, int pitch, int col0, int lane,
                                              floatx4 acc) const {
    const int g = lane >> 4, j = lane & 15;
    const bf16* base = tile + (4 * g + (j >> 2)) * pitch + col0 + 4 * (j & 3);
#pragma unroll
    for (int s = 0; s < NT16 / 2; ++s) {
      typedef __attribute__((address_space(3))) bf16x4 lds4;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)(base + (32 * s) * pitch));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)(base + (32 * s + 16) * pitch));
      bf16x8 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) { a[r] = lo[r]; a[4 + r] = hi[r]; }
      acc = Mfma16<bf16>::mma(a, f[s], acc);
    }
    return acc;
  }
  // acc += A . B where A's row (this lane's) is arow[c] over the contraction c.
  __device__ __forceinline__ floatx4 apply(const bf16* arow, int g, floatx4 acc) const {
#pragma unroll
    for (int s = 0; s < NT16 / 2; ++s) {
      const bf16x4 lo = *reinterpret_cast<const bf16x4*>(arow + (2 * s) * 16 + g * 4);
      const bf16x4 hi = *reinterpret_cast<const bf16x4*>(arow + (2 * s + 1) * 16 + g * 4);
      bf16x8 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) { a[r] = lo[r]; a[4 + r] = hi[r]; }
      acc = Mfma16<bf16>::mma(a, f[s], acc);
    }
    return acc;
  }
};
template <int NT16>
struct AccFrag<float, NT16> {
  floatx4 f[NT16];
  __device__ __forceinline__ void set(const floatx4 (&p)[NT16]) {
#pragma unroll
    for (int t = 0; t < NT16; ++t) f[t] = p[t];
  }
  __device__ __forceinline__ floatx4 apply_tr(const float*, int, int, int, floatx4 acc) const {
    return acc;   // fp32 reads explicitly transposed tiles (apply)
  }
  __device__ __forceinline__ floatx4 apply(const float* arow, int g, floatx4 acc) const {
#pragma unroll
    for (int t = 0; t < NT16; ++t) {
      const floatx4 a = *reinterpret_cast<const floatx4*>(arow + t * 16 + g * 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc = Mfma16<float>::mma(a[r], f[t][r], acc);
    }
    return acc;
  }
};

// ---------------------------------------------------------------- forward ---

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const T* __restrict__ qkv, float* __restrict__ o,
                                                       T* __restrict__ o_cast, float* __restrict__ lse,
                                                       int Tn, int H, int Hkv, int n_qblk) {
  typedef Cfg<T, HD> C;
  constexpr int BKV = C::BKV, NKT = BKV / 16, KP = HD + C::PAD, VP = BKV + C::PAD;
  __shared__ __attribute__((aligned(16))) T Ks[BKV * KP];
  __shared__ __attribute__((aligned(16))) T Vt[C::TR ? BKV * KP : HD * VP];   // bf16: V row-major

  const int qb = n_qblk - 1 - (int)blockIdx.x;   // longest rows first
  const int h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / (H / Hkv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int64_t ld = (int64_t)(H + 2 * Hkv) * HD;
  const T* base = qkv + (int64_t)b * Tn * ld;
  const T* Qg = base + h * HD;
  const T* Kg = base + (H + kvh) * HD;
  const T* Vg = base + (H + Hkv + kvh) * HD;

  const int q = qb * 64 + w * 16 + l16;
  T qf[C::HQ];
  load_frag<T, HD>(qf, Qg, ld, q, Tn, g);

  const float sl2 = LOG2E / sqrtf((float)HD);
  float m = -INFINITY, l = 0.f;
  floatx4 oacc[C::HT];
#pragma unroll
  for (int i = 0; i < C::HT; ++i) oacc[i] = floatx4{0, 0, 0, 0};

  const int q_last = min(Tn, qb * 64 + 64) - 1;
  const int n_kt = q_last / BKV + 1;
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * BKV;
    __syncthreads();
    load_rows<T, HD>(Ks, Kg, ld, k0, BKV, Tn, tid);
    if constexpr (C::TR)
      load_rows<T, HD>(Vt, Vg, ld, k0, BKV, Tn, tid);
    else
      load_rows_t<T, HD>(Vt, Vg, ld, k0, BKV, Tn, tid);
    __syncthreads();

    floatx4 s[NKT];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      s[t] = contract_hd<T, HD>(Ks + (t * 16 + l16) * KP + g * C::HQ, qf, floatx4{0, 0, 0, 0});
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + t * 16 + g * 4 + r;
        const float v = key <= q ? s[t][r] * sl2 : -INFINITY;
        s[t][r] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
    mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
    const float m_new = fmaxf(m, mx);
    const float alpha = exp2f(m - m_new);
    float rs = 0.f;
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(s[t][r] - m_new);
        s[t][r] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 16, WAVE);
    rs += __shfl_xor(rs, 32, WAVE);
    l = l * alpha + rs;
    m = m_new;
    AccFrag<T, NKT> pf;
    pf.set(s);
#pragma unroll
    for (int ht = 0; ht < C::HT; ++ht) {
      oacc[ht] *= alpha;
      if constexpr (C::TR)
        oacc[ht] = pf.apply_tr(Vt, KP, ht * 16, lane, oacc[ht]);
      else
        oacc[ht] = pf.apply(Vt + (ht * 16 + l16) * VP, g, oacc[ht]);
    }
  }

  if (q < Tn) {
    const float inv = 1.f / l;
    const int64_t row = (int64_t)b * Tn + q;
    float* orow = o + row * (int64_t)H * HD + h * HD;
#pragma unroll
    for (int ht = 0; ht < C::HT; ++ht) {
      floatx4 v = oacc[ht] * inv;
      *reinterpret_cast<floatx4*>(orow + ht * 16 + g * 4) = v;
      if (o_cast) {
        T* crow = o_cast + row * (int64_t)H * HD + h * HD + ht * 16 + g * 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) crow[r] = from_f32<T>(v[r]);
      }
    }
    if (g == 0) lse[((int64_t)b * H + h) * Tn + q] = (m + log2f(l)) * LN2;
  }
}

// --------------------------------------------------------------- backward ---

template <typename OutT>
__device__ __forceinline__ void put4(OutT* p, floatx4 v) {
  if constexpr (sizeof(OutT) == 4) {
    *reinterpret_cast<floatx4*>(p) = v;
  } else {
    bf16x4 b;
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = to_bf16(v[i]);
    *reinterpret_cast<bf16x4*>(p) = b;
  }
}

// One head's gradient row held by the 4 lanes of a column group: lane group g
// owns columns ht*16 + g*4 + r. Scaled, then (if cs is not NULL) rotated by
// the negative RoPE angle of the row's position -- the backward of the
// half-split rotation pairs column i with i + HD/2 -- and stored as OutT.
template <typename OutT, int HD>
__device__ __forceinline__ void store_grad_row(OutT* row, const floatx4 (&acc)[HD / 16], float scale,
                                               const float* cs, const float* sn, int g) {
  constexpr int HT = HD / 16, HALF = HD / 2;
  if (!cs) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) put4<OutT>(row + ht * 16 + g * 4, acc[ht] * scale);
    return;
  }
  if constexpr (HT >= 2) {
#pragma unroll
    for (int ht = 0; ht < HT / 2; ++ht) {
      const int c0 = ht * 16 + g * 4;
      const floatx4 x1 = acc[ht] * scale, x2 = acc[ht + HT / 2] * scale;
      floatx4 o1, o2;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float c = cs[c0 + r], s = sn[c0 + r];
        o1[r] = x1[r] * c + x2[r] * s;
        o2[r] = x2[r] * c - x1[r] * s;
      }
      put4<OutT>(row + c0, o1);
      put4<OutT>(row + HALF + c0, o2);
    }
  } else {
    // hd = 16: the partner column sits in the lane 32 apart (g ^ 2)
    const floatx4 x = acc[0] * scale;
    floatx4 y;
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = __shfl_xor(x[r], 32, 64);
    const bool lo = g < 2;
    const int c0 = (g & 1) * 4;   // column within the half
    floatx4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float c = cs[c0 + r], s = sn[c0 + r];
      o[r] = lo ? x[r] * c + y[r] * s : x[r] * c - y[r] * s;
    }
    put4<OutT>(row + g * 4, o);
  }
}

// D[b,h,t] = sum_i dO[m, h*HD+i] O[m, h*HD+i]; dO also rounded to T.
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(const float* __restrict__ o,
                                                           const float* __restrict__ dout,
                                                           T* __restrict__ dcast, float* __restrict__ D,
                                                           int64_t rows, int Tn, int H) {
  const int lane = threadIdx.x & 63;
  // one wave per (m, h) pair, striding over the grid
  for (int64_t rid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); rid < rows; rid += (int64_t)gridDim.x * 4) {
    const int64_t m = rid / H;
    const int h = (int)(rid % H);
    const int64_t off = m * (int64_t)H * HD + h * HD;
    float acc = 0.f;
    for (int i = lane; i < HD; i += 64) {
      const float d = dout[off + i];
      acc += d * o[off + i];
      dcast[off + i] = from_f32<T>(d);
    }
    acc = wave_sum(acc);
    if (lane == 0) {
      const int64_t b = m / Tn, t = m % Tn;
      D[(b * H + h) * Tn + t] = acc;
    }
  }
}

// dK, dV for one 64-key block of kv head kvh, summed over the query heads of
// its group and every query block at or after the diagonal.
template <typename T, int HD, typename OutT>
__global__ __launch_bounds__(256) void attn_bwd_dkv_kernel(const T* __restrict__ qkv,
                                                           const T* __restrict__ dcast,
                                                           const float* __restrict__ lse,
                                                           const float* __restrict__ D,
                                                           OutT* __restrict__ dqkv,
                                                           const float* __restrict__ rcos,
                                                           const float* __restrict__ rsin, int Tn,
                                                           int H, int Hkv) {
  typedef Cfg<T, HD> C;
  constexpr int BQ = C::BQ, NQT = BQ / 16, RP = HD + C::PAD, TP = BQ + C::PAD;
  __shared__ __attribute__((aligned(16))) T Qs[BQ * RP];
  __shared__ __attribute__((aligned(16))) T Qt[C::TR ? 8 : HD * TP];   // fp32 only
  __shared__ __attribute__((aligned(16))) T Ds[BQ * RP];
  __shared__ __attribute__((aligned(16))) T Dt[C::TR ? 8 : HD * TP];   // fp32 only
  __shared__ float lse_s[BQ], D_s[BQ];

  const int kb = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int grp = H / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int64_t ld = (int64_t)(H + 2 * Hkv) * HD, ldo = (int64_t)H * HD;
  const T* base = qkv + (int64_t)b * Tn * ld;
  const T* dbase = dcast + (int64_t)b * Tn * ldo;
  const int k0 = kb * 64;
  const int key = k0 + w * 16 + l16;   // this lane's key (column)

  T kf[C::HQ], vf[C::HQ];
  load_frag<T, HD>(kf, base + (H + kvh) * HD, ld, key, Tn, g);
  load_frag<T, HD>(vf, base + (H + Hkv + kvh) * HD, ld, key, Tn, g);

  floatx4 dk[C::HT], dv[C::HT];
#pragma unroll
  for (int i = 0; i < C::HT; ++i) dk[i] = dv[i] = floatx4{0, 0, 0, 0};
  const float sl2 = LOG2E / sqrtf((float)HD);

  const int n_qt = (Tn + BQ - 1) / BQ;
  for (int j = 0; j < grp; ++j) {
    const int h = kvh * grp + j;
    const float* lse_h = lse + ((int64_t)b * H + h) * Tn;
    const float* D_h = D + ((int64_t)b * H + h) * Tn;
    for (int qt = k0 / BQ; qt < n_qt; ++qt) {
      const int q0 = qt * BQ;
      __syncthreads();
      load_rows<T, HD>(Qs, base + h * HD, ld, q0, BQ, Tn, tid);
      load_rows<T, HD>(Ds, dbase + h * HD, ldo, q0, BQ, Tn, tid);
      if constexpr (!C::TR) {
        load_rows_t<T, HD>(Qt, base + h * HD, ld, q0, BQ, Tn, tid);
        load_rows_t<T, HD>(Dt, dbase + h * HD, ldo, q0, BQ, Tn, tid);
      }
      if (tid < BQ) {
        const bool ok = q0 + tid < Tn;
        lse_s[tid] = ok ? lse_h[q0 + tid] * LOG2E : 0.f;
        D_s[tid] = ok ? D_h[q0 + tid] : 0.f;
      }
      __syncthreads();

      floatx4 p[NQT], ds[NQT];
#pragma unroll
      for (int u = 0; u < NQT; ++u) {
        const floatx4 s = contract_hd<T, HD>(Qs + (u * 16 + l16) * RP + g * C::HQ, kf, floatx4{0, 0, 0, 0});
        const floatx4 dp = contract_hd<T, HD>(Ds + (u * 16 + l16) * RP + g * C::HQ, vf, floatx4{0, 0, 0, 0});
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qr = u * 16 + g * 4 + r;
          const int qi = q0 + qr;
          const float pv = (key <= qi && qi < Tn) ? exp2f(s[r] * sl2 - lse_s[qr]) : 0.f;
          p[u][r] = pv;
          ds[u][r] = pv * (dp[r] - D_s[qr]);
        }
      }
      AccFrag<T, NQT> pf, sf;
      pf.set(p);
      sf.set(ds);
#pragma unroll
      for (int ht = 0; ht < C::HT; ++ht) {
        if constexpr (C::TR) {
          dv[ht] = pf.apply_tr(Ds, RP, ht * 16, lane, dv[ht]);
          dk[ht] = sf.apply_tr(Qs, RP, ht * 16, lane, dk[ht]);
        } else {
          dv[ht] = pf.apply(Dt + (ht * 16 + l16) * TP, g, dv[ht]);
          dk[ht] = sf.apply(Qt + (ht * 16 + l16) * TP, g, dk[ht]);
        }
      }
    }
  }

  // lanes l and l ^ 32 (the hd = 16 rotation partners) hold the same key, so
  // both take this branch or neither does
  if (key < Tn) {
    OutT* row = dqkv + ((int64_t)b * Tn + key) * ld;   // dqkv has the qkv layout
    const float* cs = rcos ? rcos + (int64_t)key * (HD / 2) : nullptr;
    const float* sn = rsin ? rsin + (int64_t)key * (HD / 2) : nullptr;
    store_grad_row<OutT, HD>(row + (H + kvh) * HD, dk, 1.f / sqrtf((float)HD), cs, sn, g);
    store_grad_row<OutT, HD>(row + (H + Hkv + kvh) * HD, dv, 1.f, nullptr, nullptr, g);
  }
}

// dQ for one 64-query block of head h over the key tiles up to the diagonal.
template <typename T, int HD, typename OutT>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(const T* __restrict__ qkv,
                                                          const T* __restrict__ dcast,
                                                          const float* __restrict__ lse,
                                                          const float* __restrict__ D,
                                                          OutT* __restrict__ dqkv,
                                                          const float* __restrict__ rcos,
                                                          const float* __restrict__ rsin, int Tn,
                                                          int H, int Hkv, int n_qblk) {
  typedef Cfg<T, HD> C;
  constexpr int BKV = C::BKV, NKT = BKV / 16, KP = HD + C::PAD, TP = BKV + C::PAD;
  __shared__ __attribute__((aligned(16))) T Ks[BKV * KP];
  __shared__ __attribute__((aligned(16))) T Kt[C::TR ? 8 : HD * TP];   // fp32 only
  __shared__ __attribute__((aligned(16))) T Vs[BKV * KP];

  const int qb = n_qblk - 1 - (int)blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / (H / Hkv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int64_t ld = (int64_t)(H + 2 * Hkv) * HD, ldo = (int64_t)H * HD;
  const T* base = qkv + (int64_t)b * Tn * ld;
  const T* Kg = base + (H + kvh) * HD;
  const T* Vg = base + (H + Hkv + kvh) * HD;

  const int q = qb * 64 + w * 16 + l16;
  T qf[C::HQ], df[C::HQ];
  load_frag<T, HD>(qf, base + h * HD, ld, q, Tn, g);
  load_frag<T, HD>(df, dcast + (int64_t)b * Tn * ldo + h * HD, ldo, q, Tn, g);
  const bool qok = q < Tn;
  const float lse2 = qok ? lse[((int64_t)b * H + h) * Tn + q] * LOG2E : 0.f;
  const float Dq = qok ? D[((int64_t)b * H + h) * Tn + q] : 0.f;
  const float sl2 = LOG2E / sqrtf((float)HD);

  floatx4 dq[C::HT];
#pragma unroll
  for (int i = 0; i < C::HT; ++i) dq[i] = floatx4{0, 0, 0, 0};

  const int q_last = min(Tn, qb * 64 + 64) - 1;
  const int n_kt = q_last / BKV + 1;
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * BKV;
    __syncthreads();
    load_rows<T, HD>(Ks, Kg, ld, k0, BKV, Tn, tid);
    if constexpr (!C::TR) load_rows_t<T, HD>(Kt, Kg, ld, k0, BKV, Tn, tid);
    load_rows<T, HD>(Vs, Vg, ld, k0, BKV, Tn, tid);
    __syncthreads();
    floatx4 ds[NKT];
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      const floatx4 s = contract_hd<T, HD>(Ks + (t * 16 + l16) * KP + g * C::HQ, qf, floatx4{0, 0, 0, 0});
      const floatx4 dp = contract_hd<T, HD>(Vs + (t * 16 + l16) * KP + g * C::HQ, df, floatx4{0, 0, 0, 0});
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + t * 16 + g * 4 + r;
        const float pv = (key <= q && qok) ? exp2f(s[r] * sl2 - lse2) : 0.f;
        ds[t][r] = pv * (dp[r] - Dq);
      }
    }
    AccFrag<T, NKT> sf;
    sf.set(ds);
#pragma unroll
    for (int ht = 0; ht < C::HT; ++ht) {
      if constexpr (C::TR)
        dq[ht] = sf.apply_tr(Ks, KP, ht * 16, lane, dq[ht]);
      else
        dq[ht] = sf.apply(Kt + (ht * 16 + l16) * TP, g, dq[ht]);
    }
  }
  if (qok) {   // uniform across the hd = 16 rotation partners (same query)
    OutT* row = dqkv + ((int64_t)b * Tn + q) * ld + h * HD;
    const float* cs = rcos ? rcos + (int64_t)q * (HD / 2) : nullptr;
    const float* sn = rsin ? rsin + (int64_t)q * (HD / 2) : nullptr;
    store_grad_row<OutT, HD>(row, dq, 1.f / sqrtf((float)HD), cs, sn, g);
  }
}

template <typename T, int HD>
hipError_t fwd_launch(const void* qkv, float* o, void* oc, float* lse, int B, int Tn, int H, int Hkv,
                      hipStream_t s) {
  const int nq = (Tn + 63) / 64;
  hipLaunchKernelGGL((attn_fwd_kernel<T, HD>), dim3(nq, H, B), dim3(256), 0, s, (const T*)qkv, o,
                     (T*)oc, lse, Tn, H, Hkv, nq);
  return hipGetLastError();
}

template <typename T, int HD, typename OutT>
hipError_t bwd_launch(const void* qkv, const float* o, const float* dout, const float* lse,
                      void* dqkv_v, const float* rcos, const float* rsin, void* ws, int B, int Tn,
                      int H, int Hkv, hipStream_t s) {
  OutT* dqkv = static_cast<OutT*>(dqkv_v);
  const int64_t M = (int64_t)B * Tn;
  float* D = reinterpret_cast<float*>(ws);
  T* dcast = reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + attn_ws_d_bytes(B, Tn, H));
  const int64_t rows = M * H;
  hipLaunchKernelGGL((attn_bwd_pre_kernel<T, HD>), dim3((unsigned)std::min<int64_t>((rows + 3) / 4, 1 << 22)), dim3(256), 0, s,
                     o, dout, dcast, D, rows, Tn, H);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nk = (Tn + 63) / 64;
  hipLaunchKernelGGL((attn_bwd_dkv_kernel<T, HD, OutT>), dim3(nk, Hkv, B), dim3(256), 0, s,
                     (const T*)qkv, (const T*)dcast, lse, (const float*)D, dqkv, rcos, rsin, Tn, H, Hkv);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, HD, OutT>), dim3(nk, H, B), dim3(256), 0, s,
                     (const T*)qkv, (const T*)dcast, lse, (const float*)D, dqkv, rcos, rsin, Tn, H,
                     Hkv, nk);
  return hipGetLastError();
}

}  // namespace

int64_t attn_ws_d_bytes(int B, int Tn, int H) {
  return (((int64_t)B * H * Tn * 4) + 255) / 256 * 256;
}

bool attn_supported(int dtype, int hd) {
  if (dtype == 1) return hd == 64 || hd == 128;
  return hd == 16 || hd == 32 || hd == 64 || hd == 128;
}

hipError_t attn_fwd(int dtype, const void* qkv, float* o, void* o_cast, float* lse, int B, int Tn,
                    int H, int Hkv, int hd, hipStream_t s) {
  if (dtype == 1) return attn_fwd_bf16(qkv, o, o_cast, lse, B, Tn, H, Hkv, hd, s);
  switch (hd) {
    case 16: return fwd_launch<float, 16>(qkv, o, o_cast, lse, B, Tn, H, Hkv, s);
    case 32: return fwd_launch<float, 32>(qkv, o, o_cast, lse, B, Tn, H, Hkv, s);
    case 64: return fwd_launch<float, 64>(qkv, o, o_cast, lse, B, Tn, H, Hkv, s);
    default: return fwd_launch<float, 128>(qkv, o, o_cast, lse, B, Tn, H, Hkv, s);
  }
}

hipError_t attn_bwd(int dtype, const void* qkv, const float* o, const float* dout, const float* lse,
                    void* dqkv, int out_dtype, const float* rcos, const float* rsin, void* ws, int B,
                    int Tn, int H, int Hkv, int hd, hipStream_t s) {
#define MT_BWD(T, HD, O) bwd_launch<T, HD, O>(qkv, o, dout, lse, dqkv, rcos, rsin, ws, B, Tn, H, Hkv, s)
  if (dtype == 1) return attn_bwd_bf16(qkv, o, dout, lse, dqkv, out_dtype, rcos, rsin, ws, B, Tn, H, Hkv, hd, s);
  switch (hd) {
    case 16: return MT_BWD(float, 16, float);
    case 32: return MT_BWD(float, 32, float);
    case 64: return MT_BWD(float, 64, float);
    default: return MT_BWD(float, 128, float);
  }
#undef MT_BWD
}

}  // namespace mt
