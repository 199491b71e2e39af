// Matrix products of the layer template on the gfx950 matrix cores.
//
// One kernel template covers the three products of a Linear layer:
//   NT  C = A[M,K] . B[N,K]^T   forward          (A, B contiguous along K)
//   NN  C = A[M,K] . B[K,N]     input gradient   (B contiguous along N)
//   TN  C = A[K,M]^T . B[K,N]   weight gradient  (A, B contiguous along M / N)
// in fp32 (v_mfma_f32_32x32x2_f32) or bf16 with fp32 accumulation
// (v_mfma_f32_32x32x16_bf16), with an optional residual R added in the
// epilogue (C = R + A.B, R may alias C).
//
// Tiling: 128x128 output tile per 256-thread workgroup (4 wave64, 2x2, each
// 64x64 = 2x2 MFMA 32x32 tiles); the K loop moves 64 bytes per row per step
// (32 bf16 / 16 fp32) through two LDS stages. Global loads are 16-byte vectors
// along each operand's contiguous dimension; operands contiguous along M/N are
// transposed into the K-contiguous LDS layout as pairs of k rows. Inside a
// k-step, lane group g = lane/32 reads 32 contiguous bytes of its row; matrix
// core instruction s consumes slot s of those, so A and B agree on which k
// each slot holds. Workgroups are remapped so that consecutive tile ids land
// on the same XCD (each of the 8 XCDs has its own L2) and walk the output in
// groups of 8 tile rows.
#include <type_traits>

#include "dev_common.h"
#include "kernels.h"

namespace mt {
namespace {

constexpr int BM = 128, BN = 128;
constexpr int ROW_BYTES = 64;                 // k-extent of a stage per row
constexpr int PITCH = ROW_BYTES + 16;         // LDS row pitch (bytes)
constexpr int STAGE_BYTES = (BM + BN) * PITCH;

template <typename T>
struct Tile {
  static constexpr int VE = 16 / sizeof(T);   // elements per 16-byte vector
  static constexpr int BK = ROW_BYTES / sizeof(T);
};

// Load one operand tile (rows = the M or N index, ROWS = 128) for k-range
// [k0, k0 + BK) into registers.
//  KCONTIG: element (r, k) at base[(r0 + r) * ld + k]; each thread loads two
//           16-byte chunks c = tid + 256 j: row c/4, column chunk c%4.
//  otherwise: element (r, k) at base[k * ld + r0 + r]; each thread loads rows
//           k0 + 2p and k0 + 2p + 1 at 16 bytes of consecutive r.
template <typename T, bool KCONTIG>
struct Loader {
  static constexpr int VE = Tile<T>::VE;
  static constexpr int BK = Tile<T>::BK;
  Vec16 v[2];

  __device__ __forceinline__ void load(const T* __restrict__ base, int64_t ld, int r0, int rows,
                                       int k0, int K, bool vec, int tid) {
    if (KCONTIG) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = tid + 256 * j;
        const int r = c >> 2, kk = k0 + (c & 3) * VE;
        const int gr = r0 + r;
        const T* p = base + (int64_t)gr * ld + kk;
        if (vec && gr < rows && kk + VE <= K) {
          v[j] = *reinterpret_cast<const Vec16*>(p);
        } else {
          T tmp[VE];
#pragma unroll
          for (int e = 0; e < VE; ++e) tmp[e] = (gr < rows && kk + e < K) ? p[e] : T(0);
          __builtin_memcpy(&v[j], tmp, 16);
        }
      }
    } else {
      constexpr int CHUNKS = 128 / VE;       // 16-byte chunks along r
      const int p2 = tid / CHUNKS, rc = (tid % CHUNKS) * VE;
      const int gr = r0 + rc;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int kk = k0 + 2 * p2 + j;
        const T* p = base + (int64_t)kk * ld + gr;
        if (vec && kk < K && gr + VE <= rows) {
          v[j] = *reinterpret_cast<const Vec16*>(p);
        } else {
          T tmp[VE];
#pragma unroll
          for (int e = 0; e < VE; ++e) tmp[e] = (kk < K && gr + e < rows) ? p[e] : T(0);
          __builtin_memcpy(&v[j], tmp, 16);
        }
      }
    }
  }

  // Write the registers into the K-contiguous LDS tile (row pitch PITCH bytes).
  __device__ __forceinline__ void store(char* lds, int tid) const {
    if (KCONTIG) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = tid + 256 * j;
        *reinterpret_cast<Vec16*>(lds + (c >> 2) * PITCH + (c & 3) * 16) = v[j];
      }
    } else {
      constexpr int CHUNKS = 128 / VE;
      const int p2 = tid / CHUNKS, rc = (tid % CHUNKS) * VE;
      const T* a = reinterpret_cast<const T*>(&v[0]);
      const T* b = reinterpret_cast<const T*>(&v[1]);
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        T pair[2] = {a[e], b[e]};
        char* dst = lds + (rc + e) * PITCH + (2 * p2) * (int)sizeof(T);
        if (sizeof(T) == 2) {
          uint32_t u;
          __builtin_memcpy(&u, pair, 4);
          *reinterpret_cast<uint32_t*>(dst) = u;
        } else {
          uint2 u;
          __builtin_memcpy(&u, pair, 8);
          *reinterpret_cast<uint2*>(dst) = u;
        }
      }
    }
  }
};

__device__ __forceinline__ int remap_tile(int bid, int nwg) {
  // Hardware places workgroup bid on XCD bid % 8; give each XCD a contiguous
  // range of tile ids so neighbouring tiles share an L2.
  if ((nwg & 7) != 0) return bid;
  return (bid & 7) * (nwg >> 3) + (bid >> 3);
}

template <typename T, int LAYOUT>
__global__ __launch_bounds__(256) void gemm_kernel(const T* __restrict__ A, int64_t lda,
                                                   const T* __restrict__ B, int64_t ldb,
                                                   float* C, int64_t ldc, const float* R,
                                                   int64_t ldr, int M, int N, int K,
                                                   int tiles_m, int tiles_n, int vec_a,
                                                   int vec_b) {
  constexpr bool A_KC = (LAYOUT != MT_GEMM_TN);
  constexpr bool B_KC = (LAYOUT == MT_GEMM_NT);
  constexpr int BK = Tile<T>::BK;
  typedef Mfma32<T> MF;
  constexpr int KPL = BK / 2;                 // k values each lane reads per row per stage
  constexpr int NMMA = KPL / MF::KL;          // instructions per (i, j) per stage

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 5, l32 = lane & 31;

  // tile coordinates: XCD-local ids, grouped by 8 tile rows
  const int nwg = tiles_m * tiles_n;
  const int pid = remap_tile(blockIdx.x, nwg);
  const int group = 8 * tiles_n;
  const int first_m = (pid / group) * 8;
  const int gsize = min(tiles_m - first_m, 8);
  const int tm = first_m + (pid % group) % gsize;
  const int tn = (pid % group) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  Loader<T, A_KC> la;
  Loader<T, B_KC> lb;
  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{};

  const int nk = (K + BK - 1) / BK;
  if (nk > 0) {
    la.load(A, lda, m0, M, 0, K, vec_a, tid);
    lb.load(B, ldb, n0, N, 0, K, vec_b, tid);
    la.store(smem, tid);
    lb.store(smem + BM * PITCH, tid);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * STAGE_BYTES;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(A, lda, m0, M, (kt + 1) * BK, K, vec_a, tid);
      lb.load(B, ldb, n0, N, (kt + 1) * BK, K, vec_b, tid);
    }
    typename MF::frag af[2][NMMA], bfg[2][NMMA];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const char* pa = cur + (wm * 64 + i * 32 + l32) * PITCH + g * 32;
      const char* pb = cur + BM * PITCH + (wn * 64 + i * 32 + l32) * PITCH + g * 32;
      const Vec16 a0 = *reinterpret_cast<const Vec16*>(pa), a1 = *reinterpret_cast<const Vec16*>(pa + 16);
      const Vec16 b0 = *reinterpret_cast<const Vec16*>(pb), b1 = *reinterpret_cast<const Vec16*>(pb + 16);
      Vec16 av[2] = {a0, a1}, bv[2] = {b0, b1};
      __builtin_memcpy(&af[i][0], av, 32);
      __builtin_memcpy(&bfg[i][0], bv, 32);
    }
#pragma unroll
    for (int s = 0; s < NMMA; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = MF::mma(af[i][s], bfg[j][s], acc[i][j]);
    if (more) {
      char* nxt = smem + ((kt + 1) & 1) * STAGE_BYTES;
      la.store(nxt, tid);
      lb.store(nxt + BM * PITCH, tid);
    }
    __syncthreads();
  }

  // epilogue: lane holds rows (r/4)*8 + g*4 + r%4 of each 32x32 tile, column l32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + l32;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
        if (row < M) {
          float val = acc[i][j][r];
          if (R) val += R[(int64_t)row * ldr + col];
          C[(int64_t)row * ldc + col] = val;
        }
      }
    }
}

// ---------------------------------------------------------------------------
// Large-tile kernel: 256x256 output tile per 512-thread workgroup, 8 wave64 in
// 2 (M) x 4 (N), each wave owning 128x64 (4x2 MFMA 32x32 tiles); two waves per
// SIMD hide each other's latencies. The K loop moves 128 bytes per row per
// step (64 bf16 / 32 fp32) through two 64 KB LDS stages (one workgroup per
// CU). Full tiles copy each stage straight from global memory into LDS, one
// stage ahead, and read each k-step's fragments one k-step ahead of its
// products; edge tiles and K tails load through registers on a guarded path.
// LDS rows are 128 bytes with the 16-byte chunks permuted by
// S(row, c) = c ^ (row & 7) ^ ((row >> 3) & 7): fragment reads (8 consecutive
// rows, one chunk), row stores (one row, 8 chunks) and the transposed 4-byte
// stores of M/N-contiguous operands all spread over the banks.
// ---------------------------------------------------------------------------
constexpr int BIG = 256;
constexpr int BIG_THREADS = 512;
constexpr int BIG_ROW = 128;                      // bytes per LDS row
constexpr int BIG_TILE_BYTES = BIG * BIG_ROW;     // one operand tile
constexpr int BIG_STAGE = 2 * BIG_TILE_BYTES;     // A and B

__device__ __forceinline__ int swz(int row, int c) { return c ^ (row & 7) ^ ((row >> 3) & 7); }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

template <typename T, bool KCONTIG>
struct BigLoader {
  static constexpr int VE = 16 / sizeof(T);       // elements per chunk
  static constexpr int BK = BIG_ROW / sizeof(T);  // k per stage
  static constexpr int NKC = BIG * 8 / BIG_THREADS;                       // K-contiguous chunks per thread
  static constexpr int NMN = (BK / 2) * (BIG / VE) / BIG_THREADS;        // transposed tasks per thread
  static constexpr int NV = KCONTIG ? NKC : 2 * NMN;
  Vec16 v[NV];

  template <bool CHECK>
  __device__ __forceinline__ void load(const T* __restrict__ base, int64_t ld, int r0, int rows, int k0,
                                       int K, int tid) {
    if (KCONTIG) {
#pragma unroll
      for (int j = 0; j < NKC; ++j) {
        const int u = tid + BIG_THREADS * j;
        const int r = u >> 3, c = u & 7;
        const int gr = r0 + r, kk = k0 + c * VE;
        const T* p = base + (int64_t)gr * ld + kk;
        if (!CHECK || (gr < rows && kk + VE <= K)) {
          v[j] = *reinterpret_cast<const Vec16*>(p);
        } else {
          T tmp[VE];
#pragma unroll
          for (int e = 0; e < VE; ++e) tmp[e] = (gr < rows && kk + e < K) ? p[e] : T(0);
          __builtin_memcpy(&v[j], tmp, 16);
        }
      }
    } else {
      constexpr int MNC = BIG / VE;
#pragma unroll
      for (int j = 0; j < NMN; ++j) {
        const int u = tid + BIG_THREADS * j;
        const int mn_lo = u & 7, kp_lo = (u >> 3) & 7, rest = u >> 6;
        const int mnc = (rest % (MNC / 8)) * 8 + mn_lo, kp = (rest / (MNC / 8)) * 8 + kp_lo;
        const int gr = r0 + mnc * VE;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int kk = k0 + 2 * kp + h;
          const T* p = base + (int64_t)kk * ld + gr;
          if (!CHECK || (kk < K && gr + VE <= rows)) {
            v[2 * j + h] = *reinterpret_cast<const Vec16*>(p);
          } else {
            T tmp[VE];
#pragma unroll
            for (int e = 0; e < VE; ++e) tmp[e] = (kk < K && gr + e < rows) ? p[e] : T(0);
            __builtin_memcpy(&v[2 * j + h], tmp, 16);
          }
        }
      }
    }
  }

  // A K-contiguous stage straight from global memory into LDS, no register
  // staging (full tiles, k0 + BK <= K). The tile is 32 blocks of 1 KB (8
  // rows each); a global-to-LDS load writes lane l's 16 bytes at byte 16 l of
  // its block, i.e. physical chunk l % 8 of row l / 8, so each lane fetches
  // the logical chunk that the row's permutation puts there. Each wave fills
  // four blocks; completion is awaited (vmcnt) before the stage's barrier.
  __device__ __forceinline__ void direct_piece(int j, const T* __restrict__ base, int64_t ld, int r0, int k0,
                                               char* lds, int tid) const {
    static_assert(KCONTIG, "direct loads need K-contiguous rows");
    const int w = tid >> 6, lane = tid & 63;
    const int blk = w * 4 + j;
    const int r = blk * 8 + (lane >> 3);
    const int c = (lane & 7) ^ (r & 7) ^ ((r >> 3) & 7);
    copy16_to_lds(base + (int64_t)r0 * ld + k0, (uint32_t)(((int64_t)r * ld + c * VE) * (int64_t)sizeof(T)),
                  lds + blk * 1024);
  }
  __device__ __forceinline__ void direct(const T* __restrict__ base, int64_t ld, int r0, int k0, char* lds,
                                         int tid) const {
#pragma unroll
    for (int j = 0; j < BIG / 8 / (BIG_THREADS / 64); ++j) direct_piece(j, base, ld, r0, k0, lds, tid);
  }

  __device__ __forceinline__ void store(char* lds, int tid) const {
    if (KCONTIG) {
#pragma unroll
      for (int j = 0; j < NKC; ++j) {
        const int u = tid + BIG_THREADS * j;
        const int r = u >> 3, c = u & 7;
        *reinterpret_cast<Vec16*>(lds + r * BIG_ROW + (swz(r, c) << 4)) = v[j];
      }
    } else {
      constexpr int MNC = BIG / VE;
#pragma unroll
      for (int j = 0; j < NMN; ++j) {
        const int u = tid + BIG_THREADS * j;
        const int mn_lo = u & 7, kp_lo = (u >> 3) & 7, rest = u >> 6;
        const int mnc = (rest % (MNC / 8)) * 8 + mn_lo, kp = (rest / (MNC / 8)) * 8 + kp_lo;
        const int kb = 2 * kp * (int)sizeof(T);     // byte offset of the k pair in the row
        const int c = kb >> 4, off = kb & 15;
        const T* a = reinterpret_cast<const T*>(&v[2 * j]);
        const T* b = reinterpret_cast<const T*>(&v[2 * j + 1]);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          const int r = mnc * VE + e;
          T pair[2] = {a[e], b[e]};
          char* dst = lds + r * BIG_ROW + (swz(r, c) << 4) + off;
          if (sizeof(T) == 2) {
            uint32_t w;
            __builtin_memcpy(&w, pair, 4);
            *reinterpret_cast<uint32_t*>(dst) = w;
          } else {
            uint2 w;
            __builtin_memcpy(&w, pair, 8);
            *reinterpret_cast<uint2*>(dst) = w;
          }
        }
      }
    }
  }
};

// bf16 operand whose rows run along M or N (A of TN, B of NN and TN): it stays
// in its natural layout, one 512-byte LDS row per k (256 elements, 32 chunks
// of 16 bytes), chunk c of row r stored at c ^ ((r & 3) << 2). A fragment for
// 32 consecutive m (or n) and 8 consecutive k per lane group comes from two
// LDS transpose reads of 4 k each, in the k-slot order of a K-contiguous
// fragment. LDS serves the 8-byte transpose read 32 lanes (256 bytes) per
// cycle: 4 rows x 4 chunks, which the permutation puts in four different
// 64-byte bank groups, so the 32 lanes cover all 64 banks. The rows' copies
// write whole rows contiguously, conflict-free under any permutation.
struct BigNat {
  static constexpr int VE = 8;
  static constexpr int ROWB = 512;
  static constexpr int NV = 64 * 32 / BIG_THREADS;   // chunks per thread per stage
  Vec16 v[NV];
  static __device__ __forceinline__ int pchunk(int row, int c) { return c ^ ((row & 3) << 2); }

  template <bool CHECK>
  __device__ __forceinline__ void load(const bf16* __restrict__ base, int64_t ld, int r0, int rows, int k0,
                                       int K, int tid) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int q = tid + BIG_THREADS * j;
      const int row = q >> 5, c = q & 31;
      const int kk = k0 + row, gc = r0 + c * VE;
      const bf16* p = base + (int64_t)kk * ld + gc;
      if (!CHECK || (kk < K && gc + VE <= rows)) {
        v[j] = *reinterpret_cast<const Vec16*>(p);
      } else {
        bf16 tmp[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) tmp[e] = (kk < K && gc + e < rows) ? p[e] : bf16(0.f);
        __builtin_memcpy(&v[j], tmp, 16);
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int q = tid + BIG_THREADS * j;
      const int row = q >> 5, c = q & 31;
      *reinterpret_cast<Vec16*>(lds + row * ROWB + (pchunk(row, c) << 4)) = v[j];
    }
  }
  // Global -> LDS for a full stage: each wave fills four 1-KB blocks (two rows
  // each); lane l lands on physical chunk l % 32 of row l / 32 of its block and
  // fetches the logical chunk the permutation puts there.
  __device__ __forceinline__ void direct_piece(int j, const bf16* __restrict__ base, int64_t ld, int r0, int k0,
                                               char* lds, int tid) const {
    const int w = tid >> 6, lane = tid & 63;
    const int blk = w * 4 + j;
    const int row = 2 * blk + (lane >> 5);
    const int c = pchunk(row, lane & 31);
    copy16_to_lds(base + (int64_t)k0 * ld + r0, (uint32_t)(((int64_t)row * ld + c * VE) * 2), lds + blk * 1024);
  }
  __device__ __forceinline__ void direct(const bf16* __restrict__ base, int64_t ld, int r0, int k0, char* lds,
                                         int tid) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) direct_piece(j, base, ld, r0, k0, lds, tid);
  }
  // MFMA fragment: 32 consecutive m (or n) from mn0, k-step s (16 k)
  static __device__ __forceinline__ bf16x8 frag(const char* tile, int mn0, int s, int lane) {
    typedef __attribute__((address_space(3))) bf16x4 lds4;
    const int k16 = lane >> 4, i16 = lane & 15, G = lane >> 5, e = i16 >> 2, q = i16 & 3;
    const int col = mn0 + 16 * (k16 & 1) + 4 * q;
    const int row = 16 * s + 8 * G + e;                 // the second read is 4 rows on (same row & 3)
    const int off = ((pchunk(row, col >> 3)) << 4) + (col & 7) * 2;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)(tile + row * ROWB + off));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)(tile + (row + 4) * ROWB + off));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// Tile id -> (tile row, tile column): groups of 8 tile rows, column-major
// inside a group, so that concurrent workgroups share A rows and B columns.
__device__ __forceinline__ void big_tile(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group = 8 * tiles_n;
  const int first_m = (pid / group) * 8;
  const int gsize = min(tiles_m - first_m, 8);
  tm = first_m + (pid % group) % gsize;
  tn = (pid % group) / gsize;
}

// C = A B (+R) over 256x256 tiles. Workgroups [0, full_wgs) each own a tile
// over the whole K range. With ks > 1, the remaining tiles are split along K:
// workgroup full_wgs + j works on tile full_wgs + j / ks, K block j % ks (kc_k
// values each); block 0 writes C (+R), block s > 0 writes its 256x256 partial
// to ws slab (tile - full_wgs) * (ks - 1) + s - 1, for gemm_big_fixup.
template <typename T, int LAYOUT>
__global__ __launch_bounds__(BIG_THREADS, 1) void gemm_big_kernel(const T* __restrict__ A_, int64_t lda,
                                                                  const T* __restrict__ B_, int64_t ldb,
                                                                  float* C_, int64_t ldc_, const float* R_,
                                                                  int64_t ldr, int M, int N, int K_,
                                                                  int tiles_m, int tiles_n, int full_wgs, int ks,
                                                                  int kc_k, float* ws) {
  constexpr bool A_KC = (LAYOUT != MT_GEMM_TN);
  constexpr bool B_KC = (LAYOUT == MT_GEMM_NT);
  // bf16 M/N-contiguous operands stay in their natural layout (BigNat);
  // fp32 ones are transposed into K-contiguous LDS rows on the way in
  constexpr bool A_NAT = !A_KC && sizeof(T) == 2;
  constexpr bool B_NAT = !B_KC && sizeof(T) == 2;
  typedef Mfma32<T> MF;
  constexpr int BK = BIG_ROW / sizeof(T);
  constexpr int NSUB = 16 / (MF::KL * (int)sizeof(T));   // instructions per 16-byte chunk

  // one array per stage buffer: the compiler then sees that the copies in
  // flight into one stage do not alias the reads of the other
  __shared__ __attribute__((aligned(1024))) char st0[BIG_STAGE], st1[BIG_STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;       // 2 x 4 waves
  const int g = lane >> 5, l32 = lane & 31;

  int pid, split = 0;
  if ((int)blockIdx.x < full_wgs) {
    pid = remap_tile(blockIdx.x, full_wgs);
  } else {
    const int j = blockIdx.x - full_wgs;
    pid = full_wgs + j / ks;
    split = j % ks;
  }
  int tm, tn;
  big_tile(pid, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BIG, n0 = tn * BIG;
  const bool full = (m0 + BIG <= M) && (n0 + BIG <= N);
  // this workgroup's K range, operands and output
  const int k_begin = split * kc_k;
  const int K = (int)blockIdx.x < full_wgs ? K_ : min(K_ - k_begin, kc_k);
  const T* __restrict__ A = A_ + (A_KC ? (int64_t)k_begin : (int64_t)k_begin * lda);
  const T* __restrict__ B = B_ + (B_KC ? (int64_t)k_begin : (int64_t)k_begin * ldb);
  float* C = C_;
  int64_t ldc = ldc_;
  const float* R = R_;
  int ro = 0, co = 0;   // output origin (partials are tile-local)
  if (split > 0) {
    C = ws + ((int64_t)(pid - full_wgs) * (ks - 1) + split - 1) * BIG * BIG;
    ldc = BIG;
    R = nullptr;
    ro = m0;
    co = n0;
  }

  // LDS read offsets of this lane's rows (chunk added per k-step)
  int a_base[4], a_x[4], b_base[2], b_x[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wm * 128 + i * 32 + l32;
    a_base[i] = r * BIG_ROW;
    a_x[i] = (r & 7) ^ ((r >> 3) & 7);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = wn * 64 + j * 32 + l32;
    b_base[j] = BIG_TILE_BYTES + r * BIG_ROW;
    b_x[j] = (r & 7) ^ ((r >> 3) & 7);
  }

  typename std::conditional<A_NAT, BigNat, BigLoader<T, A_KC>>::type la;
  typename std::conditional<B_NAT, BigNat, BigLoader<T, B_KC>>::type lb;
  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{};

  const int nk = (K + BK - 1) / BK;
  // one stage of products from LDS; after the products of k-step s, hook(s)
  // issues part of the next stage's copies, so the copy instructions spread
  // over the stage instead of stalling every wave at its start
  auto mma_stage = [&](const char* cur, auto hook) {
    if constexpr (A_NAT || B_NAT) {
      // bf16 with a natural-layout operand: one 16-k MFMA step per s
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c = 2 * s + g;
        bf16x8 af[4], bfr[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (A_NAT) af[i] = BigNat::frag(cur, wm * 128 + i * 32, s, lane);
          else af[i] = *reinterpret_cast<const bf16x8*>(cur + a_base[i] + ((c ^ a_x[i]) << 4));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if constexpr (B_NAT) bfr[j] = BigNat::frag(cur + BIG_TILE_BYTES, wn * 64 + j * 32, s, lane);
          else bfr[j] = *reinterpret_cast<const bf16x8*>(cur + b_base[j] + ((c ^ b_x[j]) << 4));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        hook(s);
      }
      return;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = 2 * s + g;
      Vec16 av[4], bv[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = *reinterpret_cast<const Vec16*>(cur + a_base[i] + ((c ^ a_x[i]) << 4));
#pragma unroll
      for (int j = 0; j < 2; ++j) bv[j] = *reinterpret_cast<const Vec16*>(cur + b_base[j] + ((c ^ b_x[j]) << 4));
#pragma unroll
      for (int q = 0; q < NSUB; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          typename MF::frag fa;
          __builtin_memcpy(&fa, reinterpret_cast<const char*>(&av[i]) + q * sizeof(fa), sizeof(fa));
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            typename MF::frag fb;
            __builtin_memcpy(&fb, reinterpret_cast<const char*>(&bv[j]) + q * sizeof(fb), sizeof(fb));
            acc[i][j] = MF::mma(fa, fb, acc[i][j]);
          }
        }
      hook(s);
    }
  };
  auto no_hook = [](int) {};
  // The same stage with each k-step's fragments read one k-step ahead of its
  // products (two fragment sets), so only the first k-step of a stage waits
  // on LDS latency. Scheduling fences pin the order: k-step 0's reads, then
  // for each k-step s the hook's copies, the reads of k-step s + 1 and the
  // products of k-step s.
  struct Frags {
    Vec16 a[4], b[2];
  };
  auto read_frags = [&](const char* cur, int s, Frags& f) __attribute__((always_inline)) {
    const int c = 2 * s + g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (A_NAT) {
        const bf16x8 t = BigNat::frag(cur, wm * 128 + i * 32, s, lane);
        __builtin_memcpy(&f.a[i], &t, 16);
      } else {
        f.a[i] = *reinterpret_cast<const Vec16*>(cur + a_base[i] + ((c ^ a_x[i]) << 4));
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (B_NAT) {
        const bf16x8 t = BigNat::frag(cur + BIG_TILE_BYTES, wn * 64 + j * 32, s, lane);
        __builtin_memcpy(&f.b[j], &t, 16);
      } else {
        f.b[j] = *reinterpret_cast<const Vec16*>(cur + b_base[j] + ((c ^ b_x[j]) << 4));
      }
    }
  };
  auto mma_frags = [&](const Frags& f) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NSUB; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        typename MF::frag fa;
        __builtin_memcpy(&fa, reinterpret_cast<const char*>(&f.a[i]) + q * sizeof(fa), sizeof(fa));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          typename MF::frag fb;
          __builtin_memcpy(&fb, reinterpret_cast<const char*>(&f.b[j]) + q * sizeof(fb), sizeof(fb));
          acc[i][j] = MF::mma(fa, fb, acc[i][j]);
        }
      }
  };
  auto mma_stage_ahead = [&](const char* cur, auto hook) __attribute__((always_inline)) {
    Frags f0, f1;
    read_frags(cur, 0, f0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      hook(s);
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < 4) read_frags(cur, s + 1, (s & 1) ? f0 : f1);
      __builtin_amdgcn_sched_barrier(0);
      mma_frags((s & 1) ? f1 : f0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // guarded stage through registers (edge tiles, the K tail)
  auto reg_stage = [&](int k0, char* dst) {
    la.template load<true>(A, lda, m0, M, k0, K, tid);
    lb.template load<true>(B, ldb, n0, N, k0, K, tid);
    la.store(dst, tid);
    lb.store(dst + BIG_TILE_BYTES, tid);
  };

  bool done = false;
  if constexpr ((A_KC || A_NAT) && (B_KC || B_NAT)) {
    if (full) {
      // full tile with both operands loadable straight into LDS: every whole
      // stage goes global -> LDS directly, one stage ahead; a K tail runs last
      const int nkf = K / BK;
      if (nkf > 0) {
        la.direct(A, lda, m0, 0, st0, tid);
        lb.direct(B, ldb, n0, 0, st0 + BIG_TILE_BYTES, tid);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's LDS writes have landed
        __syncthreads();
      }
      auto fstage = [&](int kt, const char* cur, char* nxt) __attribute__((always_inline)) {
        const bool more = kt + 1 < nkf;
        // the last stage copies itself again into the free buffer (valid
        // memory, landed before the barrier, overwritten by any K tail): the
        // stage then has no branch and its LDS reads can move ahead of products
        const int kn = (more ? kt + 1 : kt) * BK;
        // copies early in the stage so that they land before its end, spread
        // over its first two k-steps (on the 14B shapes 3% faster for NT than
        // all in the first, with the fragments read one k-step ahead)
        constexpr int CSTEPS = 2;
        mma_stage_ahead(cur, [&](int s) {
          if (s < CSTEPS) {
#pragma unroll
            for (int j = 4 * s / CSTEPS; j < 4 * (s + 1) / CSTEPS; ++j) {
              la.direct_piece(j, A, lda, m0, kn, nxt, tid);
              lb.direct_piece(j, B, ldb, n0, kn, nxt + BIG_TILE_BYTES, tid);
            }
          }
        });
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
      };
      for (int kt = 0; kt < nkf; kt += 2) {   // buffers fixed at compile time
        fstage(kt, st0, st1);
        if (kt + 1 < nkf) fstage(kt + 1, st1, st0);
      }
      if (nkf < nk) {   // K tail (stage buffer nkf & 1 is free after the last barrier)
        char* tb = (nkf & 1) ? st1 : st0;
        reg_stage(nkf * BK, tb);
        __syncthreads();
        mma_stage(tb, no_hook);
      }
      done = true;
    }
  }
  if (!done) {
    auto load_stage = [&](int k0) {
      if (full && k0 + BK <= K) {
        la.template load<false>(A, lda, m0, M, k0, K, tid);
        lb.template load<false>(B, ldb, n0, N, k0, K, tid);
      } else {
        la.template load<true>(A, lda, m0, M, k0, K, tid);
        lb.template load<true>(B, ldb, n0, N, k0, K, tid);
      }
    };
    load_stage(0);
    la.store(st0, tid);
    lb.store(st0 + BIG_TILE_BYTES, tid);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
      const char* cur = (kt & 1) ? st1 : st0;
      const bool more = kt + 1 < nk;
      if (more) load_stage((kt + 1) * BK);
      mma_stage(cur, no_hook);
      if (more) {
        char* nxt = (kt & 1) ? st0 : st1;
        la.store(nxt, tid);
        lb.store(nxt + BIG_TILE_BYTES, tid);
      }
      __syncthreads();
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + l32;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
        if (row < M) {
          float val = acc[i][j][r];
          if (R) val += R[(int64_t)row * ldr + col];
          C[(int64_t)(row - ro) * ldc + (col - co)] = val;
        }
      }
    }
}

// C += the K-block partials of the split tiles, blocks 1 .. ks-1 in order.
// Block (t, y): tile full_wgs + t, 1024 of its elements (4 per thread).
__global__ __launch_bounds__(256) void gemm_big_fixup(float* C, int64_t ldc, const float* __restrict__ ws, int M,
                                                      int N, int tiles_m, int tiles_n, int full_wgs, int ks) {
  const int t = blockIdx.x;
  int tm, tn;
  big_tile(full_wgs + t, tiles_m, tiles_n, tm, tn);
  const int e = (blockIdx.y * 256 + threadIdx.x) * 4;   // element of the tile, row-major
  const int r = e / BIG, c = e % BIG;
  const float* p = ws + (int64_t)t * (ks - 1) * BIG * BIG + e;
  floatx4 v = *reinterpret_cast<const floatx4*>(p);
  for (int s = 1; s < ks - 1; ++s) v += *reinterpret_cast<const floatx4*>(p + (int64_t)s * BIG * BIG);
  const int row = tm * BIG + r, col = tn * BIG + c;
  if (row >= M) return;
  float* dst = C + (int64_t)row * ldc + col;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (col + q < N) dst[q] += v[q];
}

// C = R (or 0) for K = 0
__global__ void fill_kernel(float* C, int64_t ldc, const float* R, int64_t ldr, int M, int N) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)M * N) return;
  const int r = (int)(i / N), c = (int)(i % N);
  C[(int64_t)r * ldc + c] = R ? R[(int64_t)r * ldr + c] : 0.f;
}

template <typename T, int LAYOUT>
hipError_t launch(const void* A, int64_t lda, const void* B, int64_t ldb, float* C, int64_t ldc,
                  const float* R, int64_t ldr, int M, int N, int K, hipStream_t s) {
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  auto aligned = [](const void* p, int64_t ld) {
    return ((uintptr_t)p % 16 == 0) && ((ld * (int64_t)sizeof(T)) % 16 == 0);
  };
  hipLaunchKernelGGL((gemm_kernel<T, LAYOUT>), dim3(tm * tn), dim3(256), 0, s,
                     (const T*)A, lda, (const T*)B, ldb, C, ldc, R, ldr, M, N, K, tm, tn,
                     (int)aligned(A, lda), (int)aligned(B, ldb));
  return hipGetLastError();
}

// compute units of the current device (one workgroup of 512 threads each)
int gemm_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] <= 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

template <typename T, int LAYOUT>
hipError_t launch_big(const void* A, int64_t lda, const void* B, int64_t ldb, float* C, int64_t ldc,
                      const float* R, int64_t ldr, int M, int N, int K, float* ws, int64_t ws_bytes,
                      hipStream_t s) {
  const int tm = (M + BIG - 1) / BIG, tn = (N + BIG - 1) / BIG;
  const int tiles = tm * tn;
  constexpr int BK = BIG_ROW / sizeof(T);
  // the tiles of a last, at most half-full wave of workgroups (or of a grid
  // of at most half a wave) are split along K so that they fill it
  const int wave = gemm_cus();
  const int q = tiles / wave, r = tiles % wave;
  int full_wgs = tiles, ks = 1, kc_k = K;
  if (ws && r > 0 && 2 * r <= wave && (q * wave) % 8 == 0) {
    const int nk = (K + BK - 1) / BK;
    const int want = std::min(wave / r, nk / 4);       // at least 4 K stages per block
    if (want >= 2) {
      const int kb = (nk + want - 1) / want;           // K stages per block
      const int n = (nk + kb - 1) / kb;                 // non-empty blocks
      if (n >= 2 && (int64_t)r * (n - 1) * BIG * BIG * 4 <= ws_bytes) {
        full_wgs = q * wave;
        ks = n;
        kc_k = kb * BK;
      }
    }
  }
  hipLaunchKernelGGL((gemm_big_kernel<T, LAYOUT>), dim3(full_wgs + (tiles - full_wgs) * ks), dim3(BIG_THREADS), 0,
                     s, (const T*)A, lda, (const T*)B, ldb, C, ldc, R, ldr, M, N, K, tm, tn, full_wgs, ks, kc_k, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ks == 1) return e;
  hipLaunchKernelGGL(gemm_big_fixup, dim3(tiles - full_wgs, BIG * BIG / 1024), dim3(256), 0, s, C, ldc,
                     (const float*)ws, M, N, tm, tn, full_wgs, ks);
  return hipGetLastError();
}

bool big_ok(int dtype, const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M, int64_t N) {
  const int64_t es = dtype ? 2 : 4;
  // 16-byte rows, and byte offsets inside a 256-row tile within the copies' 32-bit range
  auto al = [&](const void* p, int64_t ld) {
    return ((uintptr_t)p % 16 == 0) && ((ld * es) % 16 == 0) && (int64_t)BIG * ld * es < MAX_COPY_OFFSET;
  };
  return al(A, lda) && al(B, ldb) && M >= 1 && N >= 1;
}

}  // namespace

hipError_t gemm_impl(int dtype, int layout, const void* A, int64_t lda, const void* B, int64_t ldb, float* C,
                     int64_t ldc, const float* R, int64_t ldr, int64_t M, int64_t N, int64_t K, int variant,
                     void* ws, int64_t ws_bytes, hipStream_t s);

hipError_t gemm(int dtype, int layout, const void* A, int64_t lda, const void* B, int64_t ldb,
                float* C, int64_t ldc, const float* R, int64_t ldr, int64_t M, int64_t N,
                int64_t K, hipStream_t s) {
  return gemm_impl(dtype, layout, A, lda, B, ldb, C, ldc, R, ldr, M, N, K, 0, nullptr, 0, s);
}

hipError_t gemm_variant(int dtype, int layout, const void* A, int64_t lda, const void* B, int64_t ldb,
                        float* C, int64_t ldc, const float* R, int64_t ldr, int64_t M, int64_t N,
                        int64_t K, int variant, hipStream_t s) {
  return gemm_impl(dtype, layout, A, lda, B, ldb, C, ldc, R, ldr, M, N, K, variant, nullptr, 0, s);
}

hipError_t gemm_ws(int dtype, int layout, const void* A, int64_t lda, const void* B, int64_t ldb, float* C,
                   int64_t ldc, const float* R, int64_t ldr, int64_t M, int64_t N, int64_t K, void* ws,
                   int64_t ws_bytes, hipStream_t s) {
  return gemm_impl(dtype, layout, A, lda, B, ldb, C, ldc, R, ldr, M, N, K, 0, ws, ws_bytes, s);
}

hipError_t gemm_impl(int dtype, int layout, const void* A, int64_t lda, const void* B, int64_t ldb, float* C,
                     int64_t ldc, const float* R, int64_t ldr, int64_t M, int64_t N, int64_t K, int variant,
                     void* ws, int64_t ws_bytes, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K > 0) {
    // 256x256 tiles when operands are 16-byte aligned and the grid still has
    // at least about half a wave of workgroups per CU, counting the K splits
    // of a small grid when a workspace allows them; else 128x128 tiles
    const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t nk = (K + 63) / 64;
    const int64_t splits = ws && big_tiles < gemm_cus() ? std::min<int64_t>(gemm_cus() / big_tiles, nk / 4) : 1;
    const bool use_big = variant == 2 || (variant == 0 && big_tiles * std::max<int64_t>(splits, 1) >= 128);
    float* wsf = ws_bytes > 0 ? static_cast<float*>(ws) : nullptr;
    if (use_big && big_ok(dtype, A, lda, B, ldb, M, N)) {
      const int m = (int)M, n = (int)N, k = (int)K;
      if (dtype == 1) {
        switch (layout) {
          case MT_GEMM_NT: return launch_big<bf16, MT_GEMM_NT>(A, lda, B, ldb, C, ldc, R, ldr, m, n, k, wsf, ws_bytes, s);
          case MT_GEMM_NN: return launch_big<bf16, MT_GEMM_NN>(A, lda, B, ldb, C, ldc, R, ldr, m, n, k, wsf, ws_bytes, s);
          default: return launch_big<bf16, MT_GEMM_TN>(A, lda, B, ldb, C, ldc, R, ldr, m, n, k, wsf, ws_bytes, s);
        }
      }
      switch (layout) {
        case MT_GEMM_NT: return launch_big<float, MT_GEMM_NT>(A, lda, B, ldb, C, ldc, R, ldr, m, n, k, wsf, ws_bytes, s);
        case MT_GEMM_NN: return launch_big<float, MT_GEMM_NN>(A, lda, B, ldb, C, ldc, R, ldr, m, n, k, wsf, ws_bytes, s);
        default: return launch_big<float, MT_GEMM_TN>(A, lda, B, ldb, C, ldc, R, ldr, m, n, k, wsf, ws_bytes, s);
      }
    }
  }
  if (K == 0) {
    const int64_t n = M * N;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, C, ldc, R,
                       ldr, (int)M, (int)N);
    return hipGetLastError();
  }
  const int m = (int)M, n = (int)N, k = (int)K;
  if (dtype == 1) {
    switch (layout) {
      case MT_GEMM_NT: return launch<bf16, MT_GEMM_NT>(A, lda, B, ldb, C, ldc, R, ldr, m, n, k, s);
      case MT_GEMM_NN: return launch<bf16, MT_GEMM_NN>(A, lda, B, ldb, C, ldc, R, ldr, m, n, k, s);
      default: return launch<bf16, MT_GEMM_TN>(A, lda, B, ldb, C, ldc, R, ldr, m, n, k, s);
    }
  }
  switch (layout) {
    case MT_GEMM_NT: return launch<float, MT_GEMM_NT>(A, lda, B, ldb, C, ldc, R, ldr, m, n, k, s);
    case MT_GEMM_NN: return launch<float, MT_GEMM_NN>(A, lda, B, ldb, C, ldc, R, ldr, m, n, k, s);
    default: return launch<float, MT_GEMM_TN>(A, lda, B, ldb, C, ldc, R, ldr, m, n, k, s);
  }
}

}  // namespace mt
