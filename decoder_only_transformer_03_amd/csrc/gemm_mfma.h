// bf16 GEMM on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
//   C[m][n] = sum_k A(m,k) B(n,k),  then an epilogue (epilogue.h)
//
// A(m,k) is A[m*lda + k] (k contiguous) or, with AT, A[k*lda + m]; likewise B.
// The linear layers use three forms: forward y = x W^T (A, B both
// k-contiguous), input gradient dx = dy W (B transposed), weight gradient
// dW = dy^T x (both transposed).
//
// Block tile BM x BN x 64 with 4 wavefronts in a 2 x 2 grid; each wavefront
// owns a (BM/2) x (BN/2) sub-tile of 32x32 MFMA tiles.  Operand tiles live in
// LDS as [row][64 k] bf16 with the 16-byte chunk index XOR-swizzled by the row
// (conflict-free ds_read_b128 of MFMA fragments).  A transposed operand is
// turned k-contiguous on its way into LDS: each thread loads an 8 (k) x 8 (row)
// block with eight 16-byte loads and transposes it in registers with
// v_perm_b32.  Two LDS stages: the global loads of tile k+1 are in flight while
// the MFMAs of tile k run; one barrier per k-tile.
//
// MFMA role assignment: the matrix-core "row" operand is the B tile (n) and
// the "column" operand the A tile (m), so each lane's accumulator holds four
// consecutive n of one m: the epilogue writes 4 consecutive columns per lane.
#pragma once
#include "kernels.h"

namespace gemm_mfma {

constexpr int BK = 64;

__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row ^ (row >> 3)) & 7); }

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// R rows x 64 k, k contiguous in global memory.
template <int R>
struct LoaderK {
  uint4 v[R / 32];
  __device__ __forceinline__ void load(const bf16_t* __restrict__ X, long ld, long r0, long rtot,
                                       int k, int K, int tid) {
    int c = tid & 7, rr = tid >> 3;
    bool kin = k + c * 8 < K;
#pragma unroll
    for (int i = 0; i < R / 32; ++i) {
      long row = r0 + rr + 32 * i;
      if (kin && row < rtot)
        v[i] = *reinterpret_cast<const uint4*>(X + row * ld + k + c * 8);
      else
        v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(bf16_t* s, int tid) const {
    int c = tid & 7, rr = tid >> 3;
#pragma unroll
    for (int i = 0; i < R / 32; ++i) {
      int row = rr + 32 * i;
      *reinterpret_cast<uint4*>(s + row * BK + swz(row, c) * 8) = v[i];
    }
  }
};

// R rows x 64 k, rows contiguous in global memory (X[k*ld + row]).
template <int R>
struct LoaderT {
  static constexpr int RC = R / 8;  // 8-row chunks across the tile
  uint4 v[8];
  __device__ __forceinline__ void load(const bf16_t* __restrict__ X, long ld, long r0, long rtot,
                                       int k, int K, int tid) {
    if (tid >= R) return;
    int rc = tid % RC, kg = tid / RC;
    long col = r0 + rc * 8;
    bool cin = col < rtot;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int kk = k + kg * 8 + j;
      if (cin && kk < K)
        v[j] = *reinterpret_cast<const uint4*>(X + (long)kk * ld + col);
      else
        v[j] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(bf16_t* s, int tid) const {
    if (tid >= R) return;
    int rc = tid % RC, kg = tid / RC;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const unsigned sel = (r & 1) ? 0x7632u : 0x5410u;
      uint4 o;
      o.x = __byte_perm(word(v[0], r >> 1), word(v[1], r >> 1), sel);
      o.y = __byte_perm(word(v[2], r >> 1), word(v[3], r >> 1), sel);
      o.z = __byte_perm(word(v[4], r >> 1), word(v[5], r >> 1), sel);
      o.w = __byte_perm(word(v[6], r >> 1), word(v[7], r >> 1), sel);
      int row = rc * 8 + r;
      *reinterpret_cast<uint4*>(s + row * BK + swz(row, kg) * 8) = o;
    }
  }
};

template <int R, bool T> struct Loader;
template <int R> struct Loader<R, false> : LoaderK<R> {};
template <int R> struct Loader<R, true> : LoaderT<R> {};

template <int BM, int BN, bool AT, bool BT, int EPI, typename TO>
__global__ __launch_bounds__(256, 1) void gemm_kernel(int M, int N, int K,
                                                      const bf16_t* __restrict__ A, long lda,
                                                      const bf16_t* __restrict__ B, long ldb,
                                                      EpiArgs e, int tiles_m, int tiles_n,
                                                      int kt_per_split) {
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int SM = WTM / 32, SN = WTN / 32;
  __shared__ __attribute__((aligned(16))) bf16_t smem[2][(BM + BN) * BK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // Tile order.  Workgroups are dispatched round-robin over the 8 XCDs; give
  // each XCD a contiguous range of tile ids so that tiles sharing operand
  // rows share that XCD's L2, then walk the range in groups of 8 M-tiles.
  const int ntiles = tiles_m * tiles_n;
  int pid = blockIdx.x;
  {
    int q = ntiles >> 3, r = ntiles & 7, x = pid & 7, loc = pid >> 3;
    pid = x * q + (x < r ? x : r) + loc;
  }
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int first_m = (pid / per_group) * GROUP;
  const int gsize = (tiles_m - first_m) < GROUP ? (tiles_m - first_m) : GROUP;
  const int tm = first_m + (pid % per_group) % gsize;
  const int tn = (pid % per_group) / gsize;
  const long m0 = (long)tm * BM;
  const long n0 = (long)tn * BN;

  const int nkt = (K + BK - 1) / BK;
  const int kt0 = blockIdx.y * kt_per_split;
  const int kt1 = (kt0 + kt_per_split) < nkt ? (kt0 + kt_per_split) : nkt;
  if (kt0 >= kt1) return;

  f32x16_t acc[SN][SM];
#pragma unroll
  for (int a = 0; a < SN; ++a)
#pragma unroll
    for (int b = 0; b < SM; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  Loader<BM, AT> la;
  Loader<BN, BT> lb;
  la.load(A, lda, m0, M, kt0 * BK, K, tid);
  lb.load(B, ldb, n0, N, kt0 * BK, K, tid);
  la.store(smem[0], tid);
  lb.store(smem[0] + BM * BK, tid);
  __syncthreads();

  for (int kt = kt0; kt < kt1; ++kt) {
    const int cur = (kt - kt0) & 1;
    const bool more = kt + 1 < kt1;
    if (more) {
      la.load(A, lda, m0, M, (kt + 1) * BK, K, tid);
      lb.load(B, ldb, n0, N, (kt + 1) * BK, K, tid);
    }
    const bf16_t* sA = smem[cur];
    const bf16_t* sB = smem[cur] + BM * BK;
#pragma unroll 1
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      bf16x8_t fa[SM], fb[SN];
#pragma unroll
      for (int sm = 0; sm < SM; ++sm) {
        int row = wm * WTM + sm * 32 + (lane & 31);
        fa[sm] = *reinterpret_cast<const bf16x8_t*>(sA + row * BK + swz(row, c) * 8);
      }
#pragma unroll
      for (int sn = 0; sn < SN; ++sn) {
        int row = wn * WTN + sn * 32 + (lane & 31);
        fb[sn] = *reinterpret_cast<const bf16x8_t*>(sB + row * BK + swz(row, c) * 8);
      }
#pragma unroll
      for (int sn = 0; sn < SN; ++sn)
#pragma unroll
        for (int sm = 0; sm < SM; ++sm)
          acc[sn][sm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[sn], fa[sm], acc[sn][sm], 0, 0, 0);
    }
    if (more) {
      la.store(smem[cur ^ 1], tid);
      lb.store(smem[cur ^ 1] + BM * BK, tid);
    }
    __syncthreads();
  }

  // acc[sn][sm][4i + j] is C[m][n] with m = sm*32 + lane%32 and
  // n = sn*32 + 8i + 4(lane/32) + j inside the wavefront's sub-tile.
#pragma unroll
  for (int sn = 0; sn < SN; ++sn)
#pragma unroll
    for (int sm = 0; sm < SM; ++sm) {
      const long m = m0 + wm * WTM + sm * 32 + (lane & 31);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long n = n0 + wn * WTN + sn * 32 + 8 * i + 4 * (lane >> 5);
        if (m < M && n < N) {
          float c4[4] = {acc[sn][sm][4 * i + 0], acc[sn][sm][4 * i + 1], acc[sn][sm][4 * i + 2],
                         acc[sn][sm][4 * i + 3]};
          epi_apply4<EPI, TO>(e, m, (int)n, c4);
        }
      }
    }
}

// Host side: launch one instantiation.
template <int BM, int BN, bool AT, bool BT, int EPI, typename TO>
hipError_t run(int M, int N, int K, const bf16_t* A, long lda, const bf16_t* B, long ldb,
               const EpiArgs& e, int split_k, hipStream_t s) {
  int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int nkt = (K + BK - 1) / BK;
  if (split_k < 1) split_k = 1;
  int kps = (nkt + split_k - 1) / split_k;
  int splits = (nkt + kps - 1) / kps;
  dim3 grid(tiles_m * tiles_n, splits);
  gemm_kernel<BM, BN, AT, BT, EPI, TO><<<grid, 256, 0, s>>>(M, N, K, A, lda, B, ldb, e, tiles_m,
                                                             tiles_n, kps);
  return hipGetLastError();
}

// Tile-shape choice and epilogue dispatch for one operand layout.
template <bool AT, bool BT>
hipError_t dispatch(int M, int N, int K, const bf16_t* A, long lda, const bf16_t* B, long ldb,
                    int epi, DType out_t, const EpiArgs& e, int split_k, hipStream_t s);

}  // namespace gemm_mfma

// Explicit instantiation of all tile shapes and epilogues of one layout.
#define GEMM_MFMA_DEFINE_DISPATCH(AT, BT)                                                       \
  namespace gemm_mfma {                                                                         \
  template <int BM, int BN>                                                                     \
  static hipError_t by_epi(int M, int N, int K, const bf16_t* A, long lda, const bf16_t* B,    \
                           long ldb, int epi, DType out_t, const EpiArgs& e, int sk,            \
                           hipStream_t s) {                                                     \
    switch (epi) {                                                                              \
      case EPI_STORE:                                                                           \
        return out_t == DT_BF16                                                                 \
                   ? run<BM, BN, AT, BT, EPI_STORE, bf16_t>(M, N, K, A, lda, B, ldb, e, 1, s)   \
                   : run<BM, BN, AT, BT, EPI_STORE, float>(M, N, K, A, lda, B, ldb, e, 1, s);   \
      case EPI_BIAS_GELU:                                                                       \
        return run<BM, BN, AT, BT, EPI_BIAS_GELU, bf16_t>(M, N, K, A, lda, B, ldb, e, 1, s);    \
      case EPI_RESID:                                                                           \
        return run<BM, BN, AT, BT, EPI_RESID, float>(M, N, K, A, lda, B, ldb, e, 1, s);         \
      case EPI_ACCUM:                                                                           \
        return run<BM, BN, AT, BT, EPI_ACCUM, float>(M, N, K, A, lda, B, ldb, e, 1, s);         \
      case EPI_ATOMIC:                                                                          \
        return run<BM, BN, AT, BT, EPI_ATOMIC, float>(M, N, K, A, lda, B, ldb, e, sk, s);       \
      case EPI_GELU_BWD:                                                                        \
        return run<BM, BN, AT, BT, EPI_GELU_BWD, bf16_t>(M, N, K, A, lda, B, ldb, e, 1, s);     \
      case EPI_PARTIAL:                                                                         \
        return run<BM, BN, AT, BT, EPI_PARTIAL, float>(M, N, K, A, lda, B, ldb, e, sk, s);      \
    }                                                                                           \
    return hipErrorInvalidValue;                                                                \
  }                                                                                             \
  template <>                                                                                   \
  hipError_t dispatch<AT, BT>(int M, int N, int K, const bf16_t* A, long lda, const bf16_t* B,  \
                              long ldb, int epi, DType out_t, const EpiArgs& e, int split_k,    \
                              hipStream_t s) {                                                  \
    long t256 = (long)((M + 255) / 256) * ((N + 255) / 256);                                    \
    long t256x128 = (long)((M + 255) / 256) * ((N + 127) / 128);                                \
    long t128 = (long)((M + 127) / 128) * ((N + 127) / 128);                                    \
    int bm = 128, bn = 128;                                                                     \
    long tiles = t128;                                                                          \
    if (t256 >= 384 || (epi == EPI_ATOMIC && t256 >= 16) || epi == EPI_PARTIAL) {               \
      bm = bn = 256; tiles = t256;                                                              \
    } else if (t256x128 >= 256) {                                                               \
      bm = 256; tiles = t256x128;                                                               \
    }                                                                                           \
    if (epi == EPI_ATOMIC && split_k == 0) {                                                    \
      int nkt = (K + BK - 1) / BK;                                                              \
      long want = (512 + tiles - 1) / tiles;                                                    \
      long cap = nkt / 4 > 0 ? nkt / 4 : 1;                                                     \
      split_k = (int)(want < cap ? want : cap);                                                 \
    }                                                                                           \
    if (bm == 256 && bn == 256)                                                                 \
      return by_epi<256, 256>(M, N, K, A, lda, B, ldb, epi, out_t, e, split_k, s);              \
    if (bm == 256)                                                                              \
      return by_epi<256, 128>(M, N, K, A, lda, B, ldb, epi, out_t, e, split_k, s);              \
    return by_epi<128, 128>(M, N, K, A, lda, B, ldb, epi, out_t, e, split_k, s);                \
  }                                                                                             \
  }
