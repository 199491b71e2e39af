// bf16 causal flash-attention forward on the gfx950 32x32x16 matrix cores.
//
// Same operation and rounding points as the generic forward in attention.hip
// (scaled, masked scores in fp32; online softmax in the log2 domain with one
// running maximum per 64-key tile; P rounded to bf16 before P.V; fp32 output,
// optional bf16 copy, natural-log logsumexp), laid out for throughput:
//
//  - a workgroup owns 128 queries of one head (4 waves x 32 queries), so each
//    K/V tile brought on chip serves 128 queries;
//  - 64-key K and V tiles are double buffered in LDS and copied there
//    straight from global memory: tile k+1 is in flight while tile k is
//    consumed, one barrier per tile;
//  - S^T = K Q^T runs with K rows from LDS as the A operand and the wave's 32
//    queries held in registers as B; O^T += V^T P^T takes P^T straight from
//    the S^T accumulator (the k-slots of each 16-key step are ordered as the
//    accumulator holds them) and V^T from the V tile through the LDS
//    transpose read, two 4-key reads per step;
//  - key sub-tiles that lie wholly above a wave's last query are skipped;
//  - work items are numbered so that the query blocks of one head run on the
//    same XCD (workgroup i goes to XCD i % 8) and share its L2, longest
//    blocks first.
#include "dev_common.h"
#include "kernels.h"

namespace mt {
namespace {

constexpr float F_LOG2E = 1.4426950408889634f;
constexpr float F_LN2 = 0.6931471805599453f;
constexpr int FQ = 128;   // queries per workgroup
constexpr int FK = 64;    // keys per tile
constexpr int FT = 256;   // threads

template <int HD>
struct F32Cfg {
  static constexpr int NS = HD / 16;        // 16-wide hd steps of Q K^T
  static constexpr int NH = HD / 32;        // 32-row hd sub-tiles of O^T
  static constexpr int ELEMS = FK * HD;
  static constexpr int WP = FK * HD * 2 / 1024 / (FT / 64);   // 1 KB copy pieces per wave
  // K and V tiles are stored without padding, the 16-byte chunks of row r in
  // the order chunk ^ perm(r) (perm depends on r mod 16). LDS serves 64
  // four-byte banks per cycle: 16 lanes of a 16-byte row read (16 rows, one
  // chunk) and 32 lanes of a transpose read (4 rows x 4 chunks) then fall on
  // 16 distinct chunk positions modulo 256 bytes, free of bank conflicts.
  __device__ static __forceinline__ int perm(int r) {
    if constexpr (HD == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  __device__ static __forceinline__ int at(int r, int col) { return r * HD + 8 * ((col >> 3) ^ perm(r)); }
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// max(m, x) for the running maximum of raw scores: the median of (m, x, +inf).
// The median instruction takes the matrix-core results as they are, where a
// maximum with IEEE semantics first quiets each operand (one more VALU
// instruction per score); chains of it fuse into three-operand maxima.
__device__ __forceinline__ float max_score(float m, float x) { return __builtin_amdgcn_fmed3f(m, x, INFINITY); }

// Direct global -> LDS copy (buffer form) of a 64-row K or V tile: wave w fills 1 KB pieces
// w*WP .. w*WP+WP-1, lane i landing 16 bytes at piece + 16 i; each lane
// fetches the chunk that the permuted layout puts there. Rows at or past the
// end of the sequence repeat the last row (those keys are masked).
template <int HD>
struct TileCopyF {
  typedef F32Cfg<HD> C;
  uint32_t off[C::WP];
  __device__ __forceinline__ static void piece(int w, int j, int lane, int& r, int& col) {
    const int e = (w * C::WP + j) * 512 + lane * 8;
    r = e / HD;
    col = 8 * (((e % HD) >> 3) ^ C::perm(r));
  }
  __device__ __forceinline__ void init(int64_t ld, int w, int lane) {
#pragma unroll
    for (int j = 0; j < C::WP; ++j) {
      int r, col;
      piece(w, j, lane, r, col);
      off[j] = (uint32_t)(((int64_t)r * ld + col) * 2);
    }
  }
  __device__ __forceinline__ void copy(bf16* tile, const bf16* src, int64_t ld, int k0, int Tn, int w,
                                       int lane) const {
    const char* base = reinterpret_cast<const char*>(src + (int64_t)k0 * ld);
    if (k0 + FK <= Tn) {
#pragma unroll
      for (int j = 0; j < C::WP; ++j) copy16_to_lds(base, off[j], tile + (w * C::WP + j) * 512);
    } else {
#pragma unroll
      for (int j = 0; j < C::WP; ++j) {
        int r, col;
        piece(w, j, lane, r, col);
        const int64_t o = ((int64_t)min(r, Tn - 1 - k0) * ld + col) * 2;
        copy16_to_lds(base, (uint32_t)o, tile + (w * C::WP + j) * 512);
      }
    }
  }
};

template <int HD>
__global__ __launch_bounds__(FT, 2) void attn_fwd_bf16_kernel(const bf16* __restrict__ qkv,
                                                             float* __restrict__ o,
                                                             bf16* __restrict__ o_cast,
                                                             float* __restrict__ lse, int Tn, int H,
                                                             int Hkv, int nq, int xcd_groups) {
  typedef F32Cfg<HD> C;
  // one array per buffer: the compiler then sees that the copy in flight into
  // one buffer does not alias the reads of the other and does not wait for it
  __shared__ __attribute__((aligned(1024))) bf16 K0[C::ELEMS], K1[C::ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 V0[C::ELEMS], V1[C::ELEMS];

  // work item: (head, query block), longest blocks first
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
  const int c = lane & 31, G = lane >> 5, k16 = lane >> 4, i16 = lane & 15;
  const int64_t ld = (int64_t)(H + 2 * Hkv) * HD;
  const bf16* base = qkv + (int64_t)b * Tn * ld;
  const bf16* Kg = base + (H + kvh) * HD;
  const bf16* Vg = base + (H + Hkv + kvh) * HD;

  const int wq0 = qb * FQ + w * 32;   // the wave's first query
  const int q = wq0 + c;              // this lane's query
  bf16x8 qf[C::NS];
  {
    const bf16* qrow = base + (int64_t)min(q, Tn - 1) * ld + h * HD + G * 8;
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(qrow + s * 16);
      qf[s] = q < Tn ? x : bf16x8{};
    }
  }

  const float sl2 = F_LOG2E / sqrtf((float)HD);
  float m = -INFINITY, l = 0.f;
  floatx16 oacc[C::NH];
#pragma unroll
  for (int i = 0; i < C::NH; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;

  const int q_hi = min(Tn, qb * FQ + FQ);   // end of the block's valid queries
  const int n_kt = (q_hi - 1) / FK + 1;

  TileCopyF<HD> cp;   // K and V rows share the stride
  cp.init(ld, w, lane);
  int rro[C::NS];     // K row reads: row c, hd columns 16 ss + 8 G
#pragma unroll
  for (int ss = 0; ss < C::NS; ++ss) rro[ss] = C::at(c, 16 * ss + 8 * G);
  int tro[C::NH][2];  // V transpose reads: rows 4G + i16/4 (+8), columns ht*32 + 16 (k16&1) + 4 (i16&3)
#pragma unroll
  for (int ht = 0; ht < C::NH; ++ht)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int col = ht * 32 + 16 * (k16 & 1) + 4 * (i16 & 3);
      tro[ht][hh] = C::at(4 * G + (i16 >> 2) + 8 * hh, col) + (col & 7);
    }

  auto tile = [&](int kt, const bf16* Kb, const bf16* Vb, bf16* Kn, bf16* Vn) __attribute__((always_inline)) {
    const int k0 = kt * FK;
    const bool more = kt + 1 < n_kt;
    if (more) {
      cp.copy(Kn, Kg, ld, k0 + FK, Tn, w, lane);
      cp.copy(Vn, Vg, ld, k0 + FK, Tn, w, lane);
    }

    // P^T V step kk (16 keys) of hd block ht
    auto pv_step = [&](int ht, int kk, const bf16x8& pb) __attribute__((always_inline)) {
      const bf16* p0 = Vb + 16 * kk * HD;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + tro[ht][0]));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + tro[ht][1]));
      const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      oacc[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[ht], 0, 0, 0);
    };

    if (k0 + FK - 1 <= wq0) {
      // interior tile: every key precedes every query of the wave (so none is
      // past the end): no masks, no selects; the output is rescaled before the
      // exponentials so that they share one region with the P^T V products.
      // Same arithmetic and order as the general path below.
      floatx16 s0, s1;
#pragma unroll
      for (int r = 0; r < 16; ++r) s0[r] = s1[r] = 0.f;
#pragma unroll
      for (int ss = 0; ss < C::NS; ++ss) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(Kb + rro[ss]);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(Kb + 32 * HD + rro[ss]);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ss], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ss], s1, 0, 0, 0);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = max_score(mx, s0[r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = max_score(mx, s1[r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
      const float m_new = fmaxf(m, mx * sl2);
      const float alpha = exp2f(m - m_new);
      const float nm = -m_new;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int ht = 0; ht < C::NH; ++ht)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[ht][r] *= alpha;
      }
      float rs = 0.f;
      bf16x8 pb0, pb1, pb2, pb3;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s0[r], sl2, nm));
        rs += p;
        if (r < 8) pb0[r] = to_bf16(p);
        else pb1[r - 8] = to_bf16(p);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s1[r], sl2, nm));
        rs += p;
        if (r < 8) pb2[r] = to_bf16(p);
        else pb3[r - 8] = to_bf16(p);
      }
#pragma unroll
      for (int ht = 0; ht < C::NH; ++ht) {
        pv_step(ht, 0, pb0);
        pv_step(ht, 1, pb1);
        pv_step(ht, 2, pb2);
        pv_step(ht, 3, pb3);
      }
      rs += __shfl_xor(rs, 32, WAVE);
      l = l * alpha + rs;
      m = m_new;
      if (more) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the next tile has landed
      __syncthreads();
      return;
    }

    // raw scores of the two 32-key sub-tiles (wave-uniform skip above the
    // diagonal; masking only on sub-tiles that cross it or the end). The
    // running maximum is taken on raw scores (the scale is positive, so it
    // commutes with the maximum) and the scale is folded into the exponent's FMA.
    floatx16 s[2];
    bool live[2];
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int kb = k0 + 32 * st;
      live[st] = kb <= wq0 + 31;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[st][r] = 0.f;
      if (live[st]) {
#pragma unroll
        for (int ss = 0; ss < C::NS; ++ss) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kb + 32 * st * HD + rro[ss]);
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ss], s[st], 0, 0, 0);
        }
        if (kb + 31 > wq0) {   // crosses the diagonal of some query of the wave (keys past the end too)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb + (r >> 2) * 8 + G * 4 + (r & 3);
            if (key > q) s[st][r] = -INFINITY;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = max_score(mx, s[st][r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
    const float m_new = fmaxf(m, mx * sl2);
    const float alpha = exp2f(m - m_new);
    const float nm = -m_new;
    float rs = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = live[st] ? __builtin_amdgcn_exp2f(fmaf(s[st][r], sl2, nm)) : 0.f;
        s[st][r] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 32, WAVE);
    l = l * alpha + rs;
    m = m_new;
    // the output needs rescaling only when some row's maximum moved
    const bool rescale = __any(alpha != 1.f);
    // P^T operands: 16-key step kk = 2*st + j takes accumulator slots 8j..8j+7
    bf16x8 pb0, pb1, pb2, pb3;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pb0[e] = to_bf16(s[0][e]);
      pb1[e] = to_bf16(s[0][8 + e]);
      pb2[e] = to_bf16(s[1][e]);
      pb3[e] = to_bf16(s[1][8 + e]);
    }

    // O^T += V^T P^T over four 16-key steps
#pragma unroll
    for (int ht = 0; ht < C::NH; ++ht) {
      if (rescale) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[ht][r] *= alpha;
      }
      if (live[0]) { pv_step(ht, 0, pb0); pv_step(ht, 1, pb1); }
      if (live[1]) { pv_step(ht, 2, pb2); pv_step(ht, 3, pb3); }
    }

    if (more) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the next tile has landed
    __syncthreads();
  };

  cp.copy(K0, Kg, ld, 0, Tn, w, lane);
  cp.copy(V0, Vg, ld, 0, Tn, w, lane);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int kt = 0; kt < n_kt; kt += 2) {
    tile(kt, K0, V0, K1, V1);
    if (kt + 1 < n_kt) tile(kt + 1, K1, V1, K0, V0);
  }

  if (q < Tn) {
    const float inv = 1.f / l;
    const int64_t row = (int64_t)b * Tn + q;
    float* orow = o + row * (int64_t)H * HD + h * HD;
    bf16* crow = o_cast ? o_cast + row * (int64_t)H * HD + h * HD : nullptr;
#pragma unroll
    for (int ht = 0; ht < C::NH; ++ht)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int col = ht * 32 + r4 * 8 + G * 4;
        floatx4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = oacc[ht][r4 * 4 + e] * inv;
        *reinterpret_cast<floatx4*>(orow + col) = v;
        if (crow) {
          bf16x4 cv;
#pragma unroll
          for (int e = 0; e < 4; ++e) cv[e] = to_bf16(v[e]);
          *reinterpret_cast<bf16x4*>(crow + col) = cv;
        }
      }
    if (G == 0) lse[((int64_t)b * H + h) * Tn + q] = (m + log2f(l)) * F_LN2;
  }
}

template <int HD>
hipError_t launch(const void* qkv, float* o, void* oc, float* lse, int B, int Tn, int H, int Hkv,
                  hipStream_t s) {
  const int nq = (Tn + FQ - 1) / FQ;
  const int64_t items = (int64_t)nq * H;
  const int xcd = (items % 8 == 0) && (H % 8 == 0);
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<HD>), dim3((unsigned)items, 1, B), dim3(FT), 0, s,
                     (const bf16*)qkv, o, (bf16*)oc, lse, Tn, H, Hkv, nq, xcd);
  return hipGetLastError();
}

}  // namespace

hipError_t attn_fwd_bf16(const void* qkv, float* o, void* o_cast, float* lse, int B, int Tn, int H,
                         int Hkv, int hd, hipStream_t s) {
  if (hd == 64) return launch<64>(qkv, o, o_cast, lse, B, Tn, H, Hkv, s);
  return launch<128>(qkv, o, o_cast, lse, B, Tn, H, Hkv, s);
}

}  // namespace mt
