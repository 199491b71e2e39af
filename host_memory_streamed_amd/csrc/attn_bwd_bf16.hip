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
//    LDS (copied in pieces spread over the previous tile's work); dV^T += dO^T P and dK^T += Q^T dS take P and dS from the
//    accumulators and dO^T, Q^T through the LDS transpose read. On short
//    sequences with grouped kv heads a workgroup takes one query head of the
//    group instead: the causal key blocks differ in length by up to the
//    sequence's block count, and as many times more, shorter work items
//    spread over the CUs longest first. Those write fp32 partials, and a
//    third pass sums them over the group's heads in head order.
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

#include <type_traits>

namespace mt {
namespace {

constexpr float B_LOG2E = 1.4426950408889634f;
constexpr int BT = 256;   // threads
constexpr int BW = 128;   // keys (dK/dV) or queries (dQ) per workgroup
constexpr int BS = 64;    // rows per streamed tile
// dK/dV work items are split over the query heads of a kv group up to this
// many tokens per sequence (the partials take B * min(T, DKV_SPLIT_T) * H *
// 2 hd fp32 of workspace)
constexpr int DKV_SPLIT_T = 8192;
#ifndef FENCE2
#define FENCE2 2          // steps per scheduling region in the pipelined phases
#endif
#ifndef FENCE3
#define FENCE3 4
#endif

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_b;

// A 64-row tile of HD bf16 columns in LDS, rows unpadded. The 16-byte chunks
// of row r sit in the order chunk ^ perm(r), perm depending on r mod 16 only.
// LDS serves 64 four-byte banks per cycle: a 16-byte row read takes 16 lanes
// per cycle (16 rows, one chunk) and a transpose read 32 lanes (4 rows x 4
// chunks), and the permutation gives each of those groups 16 distinct chunk
// positions modulo 256 bytes, so neither read pattern has a bank conflict.
// The tile is copied global -> LDS directly in 1 KB wave pieces whose lanes
// fetch their source chunk through the same permutation.
template <int HD>
struct Swz {
  static constexpr int NS = HD / 16;                  // 16-wide hd steps
  static constexpr int NH = HD / 32;                  // 32-row hd sub-tiles
  static constexpr int ELEMS = BS * HD;
  static constexpr int WP = BS * HD * 2 / 1024 / (BT / 64);   // 1 KB pieces per wave
  __device__ static __forceinline__ int perm(int r) {
    if constexpr (HD == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  // element offset of column col (col % 8 < 8 stays in its chunk) of row r
  __device__ static __forceinline__ int at(int r, int col) { return r * HD + 8 * ((col >> 3) ^ perm(r)) + (col & 7); }
  // row and column of the chunk that lane lands in piece j of wave w
  __device__ static __forceinline__ void piece(int w, int j, int lane, int& r, int& col) {
    const int e = (w * WP + j) * 512 + lane * 8;
    r = e / HD;
    col = 8 * (((e % HD) >> 3) ^ perm(r));
  }
};

// The per-lane source byte offsets of one tensor's tiles (row stride ld).
template <int HD>
struct TileCopy {
  typedef Swz<HD> S;
  uint32_t off[S::WP];
  __device__ __forceinline__ void init(int64_t ld, int w, int lane) {
#pragma unroll
    for (int j = 0; j < S::WP; ++j) {
      int r, col;
      S::piece(w, j, lane, r, col);
      off[j] = (uint32_t)(((int64_t)r * ld + col) * 2);
    }
  }
  // rows r0 .. r0+63 of src; rows at or past n (r0 < n) repeat row n-1, whose
  // products the callers mask. Completion: vmcnt(0), then a barrier.
  __device__ __forceinline__ void copy(bf16* tile, const bf16* src, int64_t ld, int r0, int n, int w,
                                       int lane) const {
    const char* base = reinterpret_cast<const char*>(src + (int64_t)r0 * ld);
    if (r0 + BS <= n) {
#pragma unroll
      for (int j = 0; j < S::WP; ++j) copy16_to_lds(base, off[j], tile + (w * S::WP + j) * 512);
    } else {
#pragma unroll
      for (int j = 0; j < S::WP; ++j) {
        int r, col;
        S::piece(w, j, lane, r, col);
        const int64_t o = ((int64_t)min(r, n - 1 - r0) * ld + col) * 2;
        copy16_to_lds(base, (uint32_t)o, tile + (w * S::WP + j) * 512);
      }
    }
  }
};

// Piecewise direct copy of a 64-row tile into the permuted layout (buffer
// form): piece j of wave w can be issued at any point of a tile's work, so
// the copy instructions spread over it. Rows at or past the end repeat the
// last row without a branch (the offset is pulled back by the excess rows).
template <int HD>
struct PieceCopy {
  typedef Swz<HD> S;
  static constexpr int RPP = 512 / HD;   // tile rows per 1 KB piece
  uint32_t off[S::WP];                   // source byte offset of the lane's chunk of piece j (whole tile)
  int row0;                              // tile row of the lane's chunk in piece 0 (piece j: + j*RPP)
  __device__ __forceinline__ void init(int64_t ld, int w, int lane) {
    int r, col;
#pragma unroll
    for (int j = 0; j < S::WP; ++j) {
      S::piece(w, j, lane, r, col);
      off[j] = (uint32_t)(((int64_t)r * ld + col) * 2);
    }
    S::piece(w, 0, lane, r, col);
    row0 = r;
  }
  // piece j of rows r0 .. r0+63 of src (row stride ld) into tile; rows at or
  // past n (r0 < n) repeat row n-1, whose products the callers mask
  __device__ __forceinline__ void copy(int j, bf16* tile, const bf16* src, int64_t ld, int r0, int n, int w) const {
    const int ex = max(0, row0 + j * RPP - (n - 1 - r0));
    copy16_to_lds(src + (int64_t)r0 * ld, off[j] - (uint32_t)ex * (uint32_t)(ld * 2), tile + (w * S::WP + j) * 512);
  }
};

__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// Per-lane offsets of the two transpose reads of a 16-row contraction step
// (rows 4G + 0..3 and 8 + 4G + 0..3 of a 16-row block, column block ht).
template <int HD>
struct TrOffsets {
  int o[Swz<HD>::NH][2];
  __device__ __forceinline__ void init(int lane) {
    const int k16 = lane >> 4, i16 = lane & 15, G = lane >> 5;
#pragma unroll
    for (int ht = 0; ht < Swz<HD>::NH; ++ht)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        o[ht][h] = Swz<HD>::at(4 * G + (i16 >> 2) + 8 * h, ht * 32 + 16 * (k16 & 1) + 4 * (i16 & 3));
  }
};

// A operand of a 16-row contraction step read transposed from a swizzled tile:
// lane (column ht*32 + lane%32, slot group G) receives rows row0 + 4G + 0..3
// and row0 + 8 + 4G + 0..3 of its column (row0 a multiple of 16), the slot
// order of a 32x32 accumulator's rows.
template <int HD>
__device__ __forceinline__ bf16x8 tr_operand(const bf16* tile, int row0, int ht, const TrOffsets<HD>& t) {
  const bf16* p = tile + row0 * HD;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_b*)(p + t.o[ht][0]));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_b*)(p + t.o[ht][1]));
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
  const int lane = threadIdx.x & 63;
  // one wave per (m, h) pair, striding over the grid
  for (int64_t rid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); rid < rows; rid += (int64_t)gridDim.x * 4) {
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
}

template <int HD, typename OutT>
__global__ __launch_bounds__(BT, 1) void attn_dkv_bf16_kernel(const bf16* __restrict__ qkv,
                                                             const bf16* __restrict__ dcast,
                                                             const float* __restrict__ lse,
                                                             const float* __restrict__ Dv,
                                                             OutT* __restrict__ dqkv,
                                                             const float* __restrict__ rcos,
                                                             const float* __restrict__ rsin, int Tn,
                                                             int H, int Hkv, int nkb, int xcd_groups, int hsplit,
                                                             float* __restrict__ part) {
  typedef Swz<HD> C;
  // one array per buffer: the compiler then sees that a copy in flight into
  // one buffer does not alias reads of the other and does not wait for it
  __shared__ __attribute__((aligned(1024))) bf16 Q0[C::ELEMS], Q1[C::ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 O0[C::ELEMS], O1[C::ELEMS];
  __shared__ __attribute__((aligned(16))) float Ls[2][BS];
  __shared__ __attribute__((aligned(16))) float Dsh[2][BS];

  // work item: (kv head, key block, head subset hs of hsplit), low key
  // blocks (the most queries) first
  const int id = blockIdx.x;
  int kvh, kb, hs;
  if (xcd_groups) {
    const int per = (nkb * Hkv * hsplit) >> 3;
    const int item = (id & 7) * per + (id >> 3);
    kvh = item / (nkb * hsplit);
    const int rem = item % (nkb * hsplit);
    kb = rem / hsplit;
    hs = rem % hsplit;
  } else {
    kvh = id % Hkv;
    const int rem = id / Hkv;
    kb = rem / hsplit;
    hs = rem % hsplit;
  }
  const int b = blockIdx.z;
  const int grp = H / Hkv / hsplit;   // query heads of this item
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = tid >> 6;
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

  PieceCopy<HD> cq, co;   // Q and dO tiles
  cq.init(ld, w, lane);
  co.init(ldo, w, lane);
  TrOffsets<HD> tro;
  tro.init(lane);
  int rro[C::NS];   // this lane's row-read offsets: row c, hd columns 16 ss + 8 G
#pragma unroll
  for (int ss = 0; ss < C::NS; ++ss) rro[ss] = C::at(c, 16 * ss + 8 * G);

  // query tiles at or after the block's first key, for every head of the group
  const int qt0 = (kb * BW) / BS;
  const int nqt = (Tn + BS - 1) / BS - qt0;
  const int n_it = grp * nqt;

  // tiles run over the item's grp heads from (kvh * hsplit + hs) * grp on, each over query tiles
  // qt0 .. qt0+nqt-1; (nx_h, nx_qt) is the next tile to stage, cu_qt the
  // current tile's query tile. (sh, sq0) is what the current tile stages:
  // the next tile, or itself again when there is none (into the free buffer,
  // never read).
  int nx_h = (kvh * hsplit + hs) * grp, nx_qt = qt0, cu_qt = qt0;
  int sh = nx_h, sq0 = nx_qt * BS;
  float lv = 0.f;
  auto pick_next = [&](bool more) __attribute__((always_inline)) {
    if (more) {
      sh = nx_h;
      sq0 = nx_qt * BS;
      if (++nx_qt == qt0 + nqt) {
        nx_qt = qt0;
        ++nx_h;
      }
    }
  };
  auto copy_q = [&](int j, bf16* Qn) __attribute__((always_inline)) { cq.copy(j, Qn, base + sh * HD, ld, sq0, Tn, w); };
  auto copy_o = [&](int j, bf16* On) __attribute__((always_inline)) { co.copy(j, On, dbase + sh * HD, ldo, sq0, Tn, w); };
  auto load_lv = [&]() __attribute__((always_inline)) {
    if (tid < 2 * BS) {
      const int qi = min(sq0 + (tid & (BS - 1)), Tn - 1);
      const int64_t idx = ((int64_t)b * H + sh) * Tn + qi;
      lv = tid < BS ? lse[idx] : Dv[idx];
    }
  };
  auto stash = [&](int buf) __attribute__((always_inline)) {
    if (tid < BS) Ls[buf][tid] = lv * B_LOG2E;
    else if (tid < 2 * BS) Dsh[buf][tid - BS] = lv;
  };

  constexpr int NA = 4 * C::NH;   // accumulation products per 32-query sub-tile
  // accumulation product t of a sub-tile: hd block t/4; dV with P rows
  // 0..15 / 16..31, then dK with dS rows 0..15 / 16..31
  auto amma = [&](int t, const bf16x8& a, const bf16x8& pb0, const bf16x8& pb1, const bf16x8& db0,
                  const bf16x8& db1) __attribute__((always_inline)) {
    const int ht = t >> 2;
    switch (t & 3) {
      case 0: dv[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb0, dv[ht], 0, 0, 0); break;
      case 1: dv[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb1, dv[ht], 0, 0, 0); break;
      case 2: dk[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, db0, dk[ht], 0, 0, 0); break;
      default: dk[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, db1, dk[ht], 0, 0, 0); break;
    }
  };
  // the transpose operand of product t for the sub-tile at row u*32 of a tile
  auto toper = [&](const bf16* Qb, const bf16* Ob, int u, int t) __attribute__((always_inline)) {
    return tr_operand<HD>((t & 3) < 2 ? Ob : Qb, 32 * u + 16 * (t & 1), t >> 2, tro);
  };
  // one query tile: Q and dO in (Qb, Ob), the next tile copied into (Qn, On)
  auto tile = [&](bool more, const bf16* Qb, const bf16* Ob, bf16* Qn, bf16* On, int buf)
      __attribute__((always_inline)) {
    const int q0 = cu_qt * BS;
    pick_next(more);

    // S = Q K^T and dP = dO V^T of sub-tile u (queries q0 + 32u ..)
    auto sdp = [&](int u, floatx16& s, floatx16& dp) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
      for (int ss = 0; ss < C::NS; ++ss) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Qb + 32 * u * HD + rro[ss]);
        const bf16x8 a2 = *reinterpret_cast<const bf16x8*>(Ob + 32 * u * HD + rro[ss]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[ss], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, vf[ss], dp, 0, 0, 0);
      }
    };
    // P and dS = P (dP - D) as bf16 operands; rows are queries
    // q0 + 32u + (r/4)*8 + G*4 + r%4, the column is this lane's key
    auto grads = [&](auto masked, int u, const floatx16& s, const floatx16& dp, bf16x8& pb0, bf16x8& pb1,
                     bf16x8& db0, bf16x8& db1) __attribute__((always_inline)) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int qr4 = 32 * u + r4 * 8 + G * 4;
        const floatx4 lq = *reinterpret_cast<const floatx4*>(&Ls[buf][qr4]);
        const floatx4 dq4 = *reinterpret_cast<const floatx4*>(&Dsh[buf][qr4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = r4 * 4 + e;
          float pv = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -lq[e]));
          if constexpr (decltype(masked)::value) {
            const int qi = q0 + qr4 + e;
            if (!(key <= qi && qi < Tn)) pv = 0.f;
          }
          const float dsv = pv * (dp[r] - dq4[e]);
          if (r < 8) { pb0[r] = to_bf16(pv); db0[r] = to_bf16(dsv); }
          else { pb1[r - 8] = to_bf16(pv); db1[r - 8] = to_bf16(dsv); }
        }
      }
    };

    if (q0 >= kw0 + 31 && q0 + BS <= Tn) {
      // Interior tile: both sub-tiles whole and unmasked, software-pipelined so
      // that the softmax arithmetic of one sub-tile runs while the matrix cores
      // work on the other:
      //   S0,dP0 | S1,dP1 + softmax 0 | accumulate sub-tile 0 + softmax 1 |
      //   accumulate sub-tile 1
      // Operands are read from LDS ahead of use; the steps of a phase are
      // fenced so the compiler keeps the interleaving.
      floatx16 s0, dp0, s1, dp1;
      floatx4 lq[4], dq[4];               // softmax statistics of the sub-tile in flight
      bf16x8 p00, p01, d00, d01;
      auto stats = [&](int u) __attribute__((always_inline)) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          lq[r4] = *reinterpret_cast<const floatx4*>(&Ls[buf][32 * u + r4 * 8 + G * 4]);
          dq[r4] = *reinterpret_cast<const floatx4*>(&Dsh[buf][32 * u + r4 * 8 + G * 4]);
        }
      };
      auto gelem = [&](int r, const floatx16& sv, const floatx16& dpv, bf16x8& pb0, bf16x8& pb1, bf16x8& db0,
                       bf16x8& db1) __attribute__((always_inline)) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sv[r], sl2, -lq[r >> 2][r & 3]));
        const float dsv = pv * (dpv[r] - dq[r >> 2][r & 3]);
        if (r < 8) { pb0[r] = to_bf16(pv); db0[r] = to_bf16(dsv); }
        else { pb1[r - 8] = to_bf16(pv); db1[r - 8] = to_bf16(dsv); }
      };

      // phase 1: S0, dP0; rows read two steps ahead
      bf16x8 ra[C::NS], rb[C::NS];
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        ra[ss] = *reinterpret_cast<const bf16x8*>(Qb + rro[ss]);
        rb[ss] = *reinterpret_cast<const bf16x8*>(Ob + rro[ss]);
      }
      stats(0);
      load_lv();
#pragma unroll
      for (int r = 0; r < 16; ++r) s0[r] = dp0[r] = 0.f;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ss = 0; ss < C::NS; ++ss) {
#pragma unroll
        for (int j = C::WP * ss / C::NS; j < C::WP * (ss + 1) / C::NS; ++j) copy_q(j, Qn);
        if (ss + 2 < C::NS) {
          ra[ss + 2] = *reinterpret_cast<const bf16x8*>(Qb + rro[ss + 2]);
          rb[ss + 2] = *reinterpret_cast<const bf16x8*>(Ob + rro[ss + 2]);
        }
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[ss], kf[ss], s0, 0, 0, 0);
        dp0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rb[ss], vf[ss], dp0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      bf16x8 qa[C::NS], oa[C::NS];        // sub-tile 1 rows, read two steps ahead
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        qa[ss] = *reinterpret_cast<const bf16x8*>(Qb + 32 * HD + rro[ss]);
        oa[ss] = *reinterpret_cast<const bf16x8*>(Ob + 32 * HD + rro[ss]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) s1[r] = dp1[r] = 0.f;
      __builtin_amdgcn_sched_barrier(0);
      // phase 2: S1, dP1 with softmax 0; read the sub-tile 0 transpose operands
      bf16x8 ta[NA];
#pragma unroll
      for (int ss = 0; ss < C::NS; ++ss) {
#pragma unroll
        for (int j = C::WP * ss / C::NS; j < C::WP * (ss + 1) / C::NS; ++j) copy_o(j, On);
        if (ss + 2 < C::NS) {
          qa[ss + 2] = *reinterpret_cast<const bf16x8*>(Qb + 32 * HD + rro[ss + 2]);
          oa[ss + 2] = *reinterpret_cast<const bf16x8*>(Ob + 32 * HD + rro[ss + 2]);
        }
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ss], kf[ss], s1, 0, 0, 0);
        dp1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[ss], vf[ss], dp1, 0, 0, 0);
#pragma unroll
        for (int r = 16 * ss / C::NS; r < 16 * (ss + 1) / C::NS; ++r) gelem(r, s0, dp0, p00, p01, d00, d01);
#pragma unroll
        for (int t = NA * ss / C::NS; t < NA * (ss + 1) / C::NS; ++t) ta[t] = toper(Qb, Ob, 0, t);
        if ((ss + 1) % FENCE2 == 0) __builtin_amdgcn_sched_barrier(0);
      }
      stats(1);
      __builtin_amdgcn_sched_barrier(0);
      // phase 3: accumulate sub-tile 0 with softmax 1; read the sub-tile 1 operands
      bf16x8 tb[NA], p10, p11, d10, d11;
#pragma unroll
      for (int j = 0; j < NA; ++j) {
        amma(j, ta[j], p00, p01, d00, d01);
#pragma unroll
        for (int r = 16 * j / NA; r < 16 * (j + 1) / NA; ++r) gelem(r, s1, dp1, p10, p11, d10, d11);
        tb[j] = toper(Qb, Ob, 1, j);
        if ((j + 1) % FENCE3 == 0) __builtin_amdgcn_sched_barrier(0);
      }
      // phase 4: accumulate sub-tile 1
#pragma unroll
      for (int j = 0; j < NA; ++j) amma(j, tb[j], p10, p11, d10, d11);
      wait_copies();
      stash(buf ^ 1);
    } else {
#pragma unroll
      for (int j = 0; j < C::WP; ++j) {
        copy_q(j, Qn);
        copy_o(j, On);
      }
      load_lv();
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int qs0 = q0 + 32 * u;
        if (qs0 + 31 < kw0) continue;   // every query of the sub-tile precedes the wave's keys
        floatx16 s, dp;
        sdp(u, s, dp);
        bf16x8 pb0, pb1, db0, db1;
        // masking only where the sub-tile meets the diagonal or the end
        if (qs0 < kw0 + 31 || qs0 + 31 >= Tn) grads(std::true_type{}, u, s, dp, pb0, pb1, db0, db1);
        else grads(std::false_type{}, u, s, dp, pb0, pb1, db0, db1);
#pragma unroll
        for (int t = 0; t < NA; ++t) amma(t, toper(Qb, Ob, u, t), pb0, pb1, db0, db1);
      }
      wait_copies();
      stash(buf ^ 1);
    }
    if (++cu_qt == qt0 + nqt) cu_qt = qt0;
    __syncthreads();
  };

  pick_next(true);
#pragma unroll
  for (int j = 0; j < C::WP; ++j) {
    copy_q(j, Q0);
    copy_o(j, O0);
  }
  load_lv();
  wait_copies();
  stash(0);
  __syncthreads();
  for (int it = 0; it < n_it; it += 2) {
    tile(it + 1 < n_it, Q0, O0, Q1, O1, 0);
    if (it + 1 < n_it) tile(it + 2 < n_it, Q1, O1, Q0, O0, 1);
  }

  if (key < Tn && hsplit > 1) {
    // partial row [dK | dV] of this head subset: part[b][kvh][hs][key][2 HD]
    float* prow = part + ((((int64_t)b * Hkv + kvh) * hsplit + hs) * Tn + key) * (2 * HD);
    store_acc_row<float, HD>(prow, dk, 1.f / sqrtf((float)HD), nullptr, nullptr, G);
    store_acc_row<float, HD>(prow + HD, dv, 1.f, nullptr, nullptr, G);
  } else if (key < Tn) {
    OutT* row = dqkv + ((int64_t)b * Tn + key) * ld;   // dqkv has the qkv layout
    const float* cs = rcos ? rcos + (int64_t)key * (HD / 2) : nullptr;
    const float* sn = rsin ? rsin + (int64_t)key * (HD / 2) : nullptr;
    store_acc_row<OutT, HD>(row + (H + kvh) * HD, dk, 1.f / sqrtf((float)HD), cs, sn, G);
    store_acc_row<OutT, HD>(row + (H + Hkv + kvh) * HD, dv, 1.f, nullptr, nullptr, G);
  }
}

// dK and dV rows from the partials of the dK/dV pass: the sum over the
// hsplit head subsets in order, then the dK rotation back (as store_acc_row)
// and the cast. One wave per (token, kv head); lane i holds hd columns i and
// i + HD/2, which the rotation pairs.
template <int HD, typename OutT>
__global__ __launch_bounds__(256) void attn_dkv_sum_kernel(const float* __restrict__ part, OutT* __restrict__ dqkv,
                                                           const float* __restrict__ rcos,
                                                           const float* __restrict__ rsin, int64_t rows, int Tn,
                                                           int H, int Hkv, int hsplit) {
  const int lane = threadIdx.x & 63;
  const int64_t ld = (int64_t)(H + 2 * Hkv) * HD;
  for (int64_t rid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); rid < rows; rid += (int64_t)gridDim.x * 4) {
    const int64_t m = rid / Hkv;   // token row b * Tn + t
    const int kvh = (int)(rid % Hkv);
    const int64_t b = m / Tn, t = m % Tn;
    const float* p0 = part + (((b * Hkv + kvh) * hsplit) * Tn + t) * (2 * HD);
    const int64_t pstride = (int64_t)Tn * 2 * HD;
    OutT* krow = dqkv + m * ld + (H + kvh) * HD;
    OutT* vrow = dqkv + m * ld + (H + Hkv + kvh) * HD;
    for (int i = lane; i < HD / 2; i += 64) {
      float k1 = 0.f, k2 = 0.f, v1 = 0.f, v2 = 0.f;
      for (int j = 0; j < hsplit; ++j) {
        const float* p = p0 + j * pstride;
        k1 += p[i];
        k2 += p[i + HD / 2];
        v1 += p[HD + i];
        v2 += p[HD + i + HD / 2];
      }
      if (rcos) {
        const float c = rcos[t * (HD / 2) + i], s = rsin[t * (HD / 2) + i];
        const float o1 = k1 * c + k2 * s, o2 = k2 * c - k1 * s;
        k1 = o1;
        k2 = o2;
      }
      krow[i] = from_f32<OutT>(k1);
      krow[i + HD / 2] = from_f32<OutT>(k2);
      vrow[i] = from_f32<OutT>(v1);
      vrow[i + HD / 2] = from_f32<OutT>(v2);
    }
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
  typedef Swz<HD> C;
  // one array per buffer (see the dK/dV pass)
  __shared__ __attribute__((aligned(1024))) bf16 K0[C::ELEMS], K1[C::ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 V0[C::ELEMS], V1[C::ELEMS];

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

  TileCopy<HD> ck;   // K and V rows share the stride
  ck.init(ld, w, lane);
  TrOffsets<HD> tro;
  tro.init(lane);
  int rro[C::NS];
#pragma unroll
  for (int ss = 0; ss < C::NS; ++ss) rro[ss] = C::at(c, 16 * ss + 8 * G);

  const int q_hi = min(Tn, qb * BW + BW);
  const int n_kt = (q_hi - 1) / BS + 1;
  auto tile = [&](int kt, const bf16* Kb, const bf16* Vb, bf16* Kn, bf16* Vn) __attribute__((always_inline)) {
    const int k0 = kt * BS;
    const bool more = kt + 1 < n_kt;
    if (more) {
      ck.copy(Kn, Kg, ld, k0 + BS, Tn, w, lane);
      ck.copy(Vn, Vg, ld, k0 + BS, Tn, w, lane);
    }
    if (k0 + BS - 1 <= wq0 && wq0 + 31 < Tn) {
      // interior tile: every key precedes every (valid) query of the wave; one
      // straight-line block, so that the softmax of one 32-key sub-tile can
      // overlap the other's products. Same arithmetic and order as below.
      floatx16 s0, dp0, s1, dp1;
#pragma unroll
      for (int r = 0; r < 16; ++r) s0[r] = dp0[r] = s1[r] = dp1[r] = 0.f;
#pragma unroll
      for (int ss = 0; ss < C::NS; ++ss) {
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(Kb + rro[ss]), qf[ss], s0, 0, 0, 0);
        dp0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(Vb + rro[ss]), df[ss], dp0, 0, 0, 0);
      }
#pragma unroll
      for (int ss = 0; ss < C::NS; ++ss) {
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(Kb + 32 * HD + rro[ss]), qf[ss], s1,
                                                     0, 0, 0);
        dp1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(Vb + 32 * HD + rro[ss]), df[ss],
                                                      dp1, 0, 0, 0);
      }
      auto grads = [&](const floatx16& sv, const floatx16& dpv, bf16x8& db0, bf16x8& db1) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sv[r], sl2, -lse2));
          const float dsv = pv * (dpv[r] - Dq);
          if (r < 8) db0[r] = to_bf16(dsv);
          else db1[r - 8] = to_bf16(dsv);
        }
      };
      bf16x8 e0, e1, f0, f1;
      grads(s0, dp0, e0, e1);
#pragma unroll
      for (int ht = 0; ht < C::NH; ++ht) {
        dq[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<HD>(Kb, 0, ht, tro), e0, dq[ht], 0, 0, 0);
        dq[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<HD>(Kb, 16, ht, tro), e1, dq[ht], 0, 0, 0);
      }
      grads(s1, dp1, f0, f1);
#pragma unroll
      for (int ht = 0; ht < C::NH; ++ht) {
        dq[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<HD>(Kb, 32, ht, tro), f0, dq[ht], 0, 0, 0);
        dq[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<HD>(Kb, 48, ht, tro), f1, dq[ht], 0, 0, 0);
      }
      if (more) wait_copies();
      __syncthreads();
      return;
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int kb0 = k0 + 32 * st;
      if (kb0 > wq0 + 31) continue;   // every key of the sub-tile follows the wave's queries
      floatx16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
      for (int ss = 0; ss < C::NS; ++ss) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kb + 32 * st * HD + rro[ss]);
        const bf16x8 a2 = *reinterpret_cast<const bf16x8*>(Vb + 32 * st * HD + rro[ss]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ss], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, df[ss], dp, 0, 0, 0);
      }
      // rows are keys kb0 + (r/4)*8 + G*4 + r%4, the column is this lane's
      // query; masking only where the sub-tile meets the diagonal or the end
      bf16x8 db0, db1;
      auto grads = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -lse2));
          if constexpr (decltype(masked)::value) {
            const int kk = kb0 + (r >> 2) * 8 + G * 4 + (r & 3);
            if (!(kk <= q && q < Tn)) pv = 0.f;
          }
          const float dsv = pv * (dp[r] - Dq);
          if (r < 8) db0[r] = to_bf16(dsv);
          else db1[r - 8] = to_bf16(dsv);
        }
      };
      if (kb0 + 31 > wq0 || wq0 + 31 >= Tn) grads(std::true_type{});
      else grads(std::false_type{});
#pragma unroll
      for (int ht = 0; ht < C::NH; ++ht) {
        dq[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<HD>(Kb, 32 * st, ht, tro), db0, dq[ht], 0, 0, 0);
        dq[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<HD>(Kb, 32 * st + 16, ht, tro), db1, dq[ht], 0, 0, 0);
      }
    }
    if (more) wait_copies();
    __syncthreads();
  };

  ck.copy(K0, Kg, ld, 0, Tn, w, lane);
  ck.copy(V0, Vg, ld, 0, Tn, w, lane);
  wait_copies();
  __syncthreads();
  for (int kt = 0; kt < n_kt; kt += 2) {
    tile(kt, K0, V0, K1, V1);
    if (kt + 1 < n_kt) tile(kt + 1, K1, V1, K0, V0);
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
  hipLaunchKernelGGL((attn_pre_bf16_kernel<HD>), dim3((unsigned)std::min<int64_t>((rows + 3) / 4, 1 << 22)), dim3(256), 0, s, o, dout,
                     dcast, D, rows, Tn, H);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb = (Tn + BW - 1) / BW;
  const int hsplit = attn_dkv_hsplit(Tn, H, Hkv);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(dcast) + (int64_t)B * Tn * H * HD * 2);
  const int64_t kv_items = (int64_t)nb * Hkv * hsplit, q_items = (int64_t)nb * H;
  hipLaunchKernelGGL((attn_dkv_bf16_kernel<HD, OutT>), dim3((unsigned)kv_items, 1, B), dim3(BT), 0, s,
                     (const bf16*)qkv, (const bf16*)dcast, lse, (const float*)D, (OutT*)dqkv, rcos, rsin,
                     Tn, H, Hkv, nb, (int)((kv_items % 8 == 0) && (Hkv % 8 == 0)), hsplit, part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (hsplit > 1) {
    const int64_t sum_rows = M * Hkv;
    hipLaunchKernelGGL((attn_dkv_sum_kernel<HD, OutT>), dim3((unsigned)std::min<int64_t>((sum_rows + 3) / 4, 1 << 22)),
                       dim3(256), 0, s, (const float*)part, (OutT*)dqkv, rcos, rsin, sum_rows, Tn, H, Hkv, hsplit);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((attn_dq_bf16_kernel<HD, OutT>), dim3((unsigned)q_items, 1, B), dim3(BT), 0, s,
                     (const bf16*)qkv, (const bf16*)dcast, lse, (const float*)D, (OutT*)dqkv, rcos, rsin,
                     Tn, H, Hkv, nb, (int)((q_items % 8 == 0) && (H % 8 == 0)));
  return hipGetLastError();
}

}  // namespace

// Head subsets per dK/dV work item: every query head of a kv group on its own
// for short sequences with grouped kv heads, else one subset.
int attn_dkv_hsplit(int Tn, int H, int Hkv) { return (H > Hkv && Tn <= DKV_SPLIT_T) ? H / Hkv : 1; }

int64_t attn_dkv_part_bytes(int B, int Tn, int H, int hd) {
  return (int64_t)B * std::min(Tn, DKV_SPLIT_T) * H * 2 * hd * 4;
}

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
