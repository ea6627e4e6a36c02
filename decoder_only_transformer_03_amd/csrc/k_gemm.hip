// GEMM entry: fp32 operands run on a vector-ALU tiled kernel (fp32 mode),
// bf16 operands on the matrix-core kernel (gemm_mfma.h).
#include <cstring>

#include "kernels.h"

namespace gemm_mfma {
template <bool AT, bool BT>
hipError_t dispatch(int M, int N, int K, const bf16_t* A, long lda, const bf16_t* B, long ldb,
                    int epi, DType out_t, const EpiArgs& e, int split_k, hipStream_t s);
}

// fp32 C[m][n] = sum_k A(m,k) B(n,k): 64 x 64 tile, 16-deep k steps through
// LDS, each thread a 4 x 4 block of C with 4 consecutive n.
template <bool AT, bool BT, int EPI, typename TO>
__global__ __launch_bounds__(256) void gemm_f32_kernel(int M, int N, int K,
                                                       const float* __restrict__ A, long lda,
                                                       const float* __restrict__ B, long ldb,
                                                       EpiArgs e, int kchunk) {
  __shared__ float As[16][68];
  __shared__ float Bs[16][68];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const long m0 = (long)blockIdx.z * 64;
  const long n0 = (long)blockIdx.x * 64;
  const int kb = blockIdx.y * kchunk;  // split-K slice (the epilogue reads blockIdx.y)
  const int ke = kb + kchunk < K ? kb + kchunk : K;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = kb; k0 < ke; k0 += 16) {
    for (int i = tid; i < 1024; i += 256) {
      int r, kk;
      if (AT) { r = i & 63; kk = i >> 6; } else { kk = i & 15; r = i >> 4; }
      long m = m0 + r;
      int k = k0 + kk;
      As[kk][r] = (m < M && k < ke) ? (AT ? A[(long)k * lda + m] : A[m * lda + k]) : 0.f;
      if (BT) { r = i & 63; kk = i >> 6; } else { kk = i & 15; r = i >> 4; }
      long n = n0 + r;
      k = k0 + kk;
      Bs[kk][r] = (n < N && k < ke) ? (BT ? B[(long)k * ldb + n] : B[n * ldb + k]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
  if constexpr (EPI == EPI_LSE) {
    // the 16 threads of one ty (lanes 16 ty .. 16 ty + 15 of a wavefront)
    // hold the 64 columns of the tile's rows ty*4 .. ty*4+3
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long m = m0 + ty * 4 + i;
      const long n = n0 + tx * 4;
      float x[4], mx = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = n + j < N ? e.alpha * acc[i][j] : -__builtin_inff();
        mx = fmaxf(mx, x[j]);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) sum += n + j < N ? __expf(x[j] - mx) : 0.f;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) sum += __shfl_xor(sum, o, 64);
      if (m < M) {
        if (tx == 0) {
          float* p = e.part + 2 * (m * e.nblk + n0 / 64);
          p[0] = mx;
          p[1] = sum;
        }
        const long c = e.tgt[m] - e.col0 - n;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (c == j && n + j < N) e.tlogit[m] = x[j];
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    long m = m0 + ty * 4 + i;
    long n = n0 + tx * 4;
    if (m < M && n < N) epi_apply4<EPI, TO>(e, m, (int)n, acc[i], blockIdx.y);
  }
}

template <bool AT, bool BT, int EPI>
static hipError_t f32_run(int M, int N, int K, const float* A, long lda, const float* B, long ldb,
                          const EpiArgs& e, int split_k, hipStream_t s) {
  if (split_k < 1) split_k = 1;
  int kchunk = (K + split_k - 1) / split_k;
  kchunk = (kchunk + 15) / 16 * 16;
  int splits = (K + kchunk - 1) / kchunk;
  dim3 grid((N + 63) / 64, splits, (M + 63) / 64);
  gemm_f32_kernel<AT, BT, EPI, float><<<grid, 256, 0, s>>>(M, N, K, A, lda, B, ldb, e, kchunk);
  return hipGetLastError();
}

template <bool AT, bool BT>
static hipError_t f32_by_epi(int M, int N, int K, const float* A, long lda, const float* B,
                             long ldb, int epi, const EpiArgs& e, int split_k, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return f32_run<AT, BT, EPI_STORE>(M, N, K, A, lda, B, ldb, e, 1, s);
    case EPI_BIAS: return f32_run<AT, BT, EPI_BIAS>(M, N, K, A, lda, B, ldb, e, 1, s);
    case EPI_BIAS_GELU: return f32_run<AT, BT, EPI_BIAS_GELU>(M, N, K, A, lda, B, ldb, e, 1, s);
    case EPI_RESID: return f32_run<AT, BT, EPI_RESID>(M, N, K, A, lda, B, ldb, e, 1, s);
    case EPI_ACCUM: return f32_run<AT, BT, EPI_ACCUM>(M, N, K, A, lda, B, ldb, e, 1, s);
    case EPI_ATOMIC: {
      if (split_k == 0) {
        long tiles = (long)((M + 63) / 64) * ((N + 63) / 64);
        long want = (512 + tiles - 1) / tiles, cap = K / 64 > 0 ? K / 64 : 1;
        split_k = (int)(want < cap ? want : cap);
      }
      return f32_run<AT, BT, EPI_ATOMIC>(M, N, K, A, lda, B, ldb, e, split_k, s);
    }
    case EPI_GELU_BWD: return f32_run<AT, BT, EPI_GELU_BWD>(M, N, K, A, lda, B, ldb, e, 1, s);
    case EPI_PARTIAL: return f32_run<AT, BT, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, e, split_k, s);
    case EPI_LSE: return f32_run<AT, BT, EPI_LSE>(M, N, K, A, lda, B, ldb, e, 1, s);
    case EPI_DLOGITS: return f32_run<AT, BT, EPI_DLOGITS>(M, N, K, A, lda, B, ldb, e, 1, s);
  }
  return hipErrorInvalidValue;
}

// Split count of a weight-gradient GEMM (long contraction, small output):
// enough K-slices that the 256x256 (bf16) or 64x64 (fp32) tiles fill the
// GPU once, each slice at least 4 k-tiles deep.
// The number of slices a launch with `s` requested actually produces (the
// launchers round the slice depth up to whole k-tiles).
static int exact_splits(DType in_t, int K, int s) {
  if (s <= 1) return 1;
  if (in_t == DT_BF16) {
    int nkt = (K + 63) / 64;
    int kps = (nkt + s - 1) / s;
    return (nkt + kps - 1) / kps;
  }
  int kchunk = ((K + s - 1) / s + 15) / 16 * 16;
  return (K + kchunk - 1) / kchunk;
}

int gemm_partial_splits(DType in_t, int M, int N, int K) {
  const int tile = in_t == DT_BF16 ? 256 : 64;
  const int kt = in_t == DT_BF16 ? 64 : 16;
  long tiles = (long)((M + tile - 1) / tile) * ((N + tile - 1) / tile);
  long s = 256 / tiles;
  long cap = (K / kt) / 4;
  if (s > cap) s = cap;
  if (s > 64) s = 64;
  return exact_splits(in_t, K, s < 1 ? 1 : (int)s);
}

// out[m*ldo + n] += sum_z part[z][m][n]  (store: out = ...)
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int splits, long MN, int N,
                                                            float* __restrict__ out, long ldo,
                                                            int store) {
  long i4 = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= MN) return;
  float4 a = *reinterpret_cast<const float4*>(part + i4);
  for (int z = 1; z < splits; ++z) {
    float4 b = *reinterpret_cast<const float4*>(part + (long)z * MN + i4);
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
  }
  long m = i4 / N;
  int n = (int)(i4 - m * N);
  float4* o = reinterpret_cast<float4*>(out + m * ldo + n);
  if (store) {
    *o = a;
    return;
  }
  float4 c = *o;
  *o = make_float4(c.x + a.x, c.y + a.y, c.z + a.z, c.w + a.w);
}

hipError_t launch_gemm_wgrad(DType in_t, int M, int N, int K, const void* A, long lda, bool a_t,
                             const void* B, long ldb, bool b_t, float* out, long ldo, float alpha,
                             float* part, long part_elems, hipStream_t s, bool store) {
  const int acc = store ? EPI_STORE : EPI_ACCUM;
  int S = gemm_partial_splits(in_t, M, N, K);
  while (S > 1 && (long)S * M * N > part_elems) S = exact_splits(in_t, K, S - 1);
  EpiArgs e;
  memset(&e, 0, sizeof(e));
  e.alpha = alpha;
  if (S == 1) {
    e.out = out;
    e.ldo = ldo;
    // Whole rounds of 256 x 256 tiles leave a last, partly idle round when
    // the tile count is not a multiple of the workgroup slots (the tied
    // lm_head: 197 x 3 tiles).  Then the leading rows run as whole rounds and
    // the remaining rows as split-K slices that fill one more round.
    if (in_t == DT_BF16 && K % 64 == 0) {
      const long slots = gemm_slots();
      const int tn = (N + 255) / 256, tm = (M + 255) / 256;
      const long tiles = (long)tm * tn, rounds = tiles / slots, tail = tiles - rounds * slots;
      const int nkt = K / 64;
      const int M1 = (int)((rounds * slots) / tn) * 256;
      if (rounds >= 1 && tail > 0 && tail * 10 < slots * 8 && nkt >= 32 && M1 > 0 && M1 < M) {
        hipError_t r = launch_gemm(in_t, M1, N, K, A, lda, a_t, B, ldb, b_t, acc, DT_F32, e, 1, s);
        if (r != hipSuccess) return r;
        const int M2 = M - M1;
        const bf16_t* A2 = reinterpret_cast<const bf16_t*>(A) + (a_t ? (long)M1 : (long)M1 * lda);
        const long tiles2 = (long)((M2 + 255) / 256) * tn;
        int S2 = (int)(slots / tiles2);
        if (S2 > nkt / 4) S2 = nkt / 4;
        S2 = exact_splits(in_t, K, S2 < 1 ? 1 : S2);
        while (S2 > 1 && (long)S2 * M2 * N > part_elems) S2 = exact_splits(in_t, K, S2 - 1);
        EpiArgs e2 = e;
        e2.out = out + (long)M1 * ldo;
        if (S2 == 1)
          return launch_gemm(in_t, M2, N, K, A2, lda, a_t, B, ldb, b_t, acc, DT_F32, e2, 1, s);
        e2.out = part;
        e2.ldo = N;
        e2.split_stride = (long)M2 * N;
        r = launch_gemm(in_t, M2, N, K, A2, lda, a_t, B, ldb, b_t, EPI_PARTIAL, DT_F32, e2, S2, s);
        if (r != hipSuccess) return r;
        const long MN2 = (long)M2 * N;
        splitk_reduce_kernel<<<(unsigned)((MN2 / 4 + 255) / 256), 256, 0, s>>>(
            part, S2, MN2, N, out + (long)M1 * ldo, ldo, store ? 1 : 0);
        return hipGetLastError();
      }
    }
    return launch_gemm(in_t, M, N, K, A, lda, a_t, B, ldb, b_t, acc, DT_F32, e, 1, s);
  }
  e.out = part;
  e.ldo = N;
  e.split_stride = (long)M * N;
  hipError_t r = launch_gemm(in_t, M, N, K, A, lda, a_t, B, ldb, b_t, EPI_PARTIAL, DT_F32, e, S, s);
  if (r != hipSuccess) return r;
  long MN = (long)M * N;
  splitk_reduce_kernel<<<(unsigned)((MN / 4 + 255) / 256), 256, 0, s>>>(part, S, MN, N, out, ldo,
                                                                          store ? 1 : 0);
  return hipGetLastError();
}

// out = epilogue(sum_z part[z]) per group of 4 columns, slices summed in
// order z = 0, 1, ... (deterministic).
template <int EPI, typename TO>
__global__ __launch_bounds__(256) void splitk_epi_kernel(const float* __restrict__ part, int splits,
                                                         int M, int N, EpiArgs e) {
  const long g = (long)blockIdx.x * 256 + threadIdx.x;  // group of 4 columns
  const int gpr = N / 4;
  if (g >= (long)M * gpr) return;
  const long m = g / gpr;
  const int n = (int)(g - m * gpr) * 4;
  const long MN = (long)M * N;
  float4 a = *reinterpret_cast<const float4*>(part + m * N + n);
  for (int z = 1; z < splits; ++z) {
    const float4 b = *reinterpret_cast<const float4*>(part + z * MN + m * N + n);
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
  }
  const float c[4] = {a.x, a.y, a.z, a.w};
  epi_apply4<EPI, TO>(e, m, n, c, 0);
}

// Few rows (M <= 16: a decoding step's batch): C = A B^T with A (M x K) and
// B (N x K) both k-contiguous bf16.  The work is streaming B once.  A
// workgroup owns CT tiles of 16 output columns; its 16 wavefronts take tile
// w % CT and split K into 16/CT contiguous ranges of 32-deep chunks, whose
// loads are all issued before their matrix products
// (v_mfma_f32_16x16x32_bf16: lane l supplies row l%16 of A and of B at
// contraction slots 8(l/16) .. +7; rows of A past M are zeros, columns past N
// read column N-1 and are dropped).  The partial 16 x 16 blocks of a tile are
// added in a fixed order through LDS, and 4 threads per row and tile apply
// the epilogue to four columns each, its inputs (residual, bias) fetched
// before the products.
constexpr int SKINNY_M = 16, SKINNY_WAVES = 16, SKINNY_BATCH = 8;
// LNA: A is LayerNorm(x) of fp32 rows x (M x K, row stride K) with weight
// lnw and bias lnb ("The Block: pre-LN and residuals"), formed here instead
// of by a separate pass, after the first chunks of B are in flight:
// wavefront w holds row w in registers and normalises it in the same order
// and arithmetic as layernorm_fwd_kernel (per-lane sums of 4-column chunks,
// then a wavefront sum; biased variance, eps 1e-5), writing it as bf16 to
// LDS, from where the fragments are read.
template <int EPI, typename TO, bool LNA, int CT>
__global__ __launch_bounds__(SKINNY_WAVES * 64) void gemm_skinny_kernel(
    int M, int N, int K, const bf16_t* __restrict__ A, long lda, const bf16_t* __restrict__ B,
    long ldb, EpiArgs e, const float* __restrict__ x, const float* __restrict__ lnw,
    const float* __restrict__ lnb) {
  constexpr int NKS = SKINNY_WAVES / CT;  // K ranges per column tile
  __shared__ float red[SKINNY_WAVES][SKINNY_M * 16];
  extern __shared__ __attribute__((aligned(16))) bf16_t sA[];  // LNA: M x K
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int ct = w % CT, ks = w / CT;
  const int n0 = (blockIdx.x * CT + ct) * 16;
  const int r = lane & 15, kq = 8 * (lane >> 4);
  const bool arow = r < M;
  const int bn = n0 + r < N ? n0 + r : N - 1;
  const bf16_t* bp = B + (long)bn * ldb + kq;
  const int nk = K / 32;
  const int c0 = (ks * nk) / NKS, c1 = ((ks + 1) * nk) / NKS;
  // Every batch runs all SKINNY_BATCH products, those of chunks past c1 on
  // zero operands (adding exactly nothing): a matrix product ignores the
  // exec mask, so none is placed under a condition.
  bf16x8_t bfv[SKINNY_BATCH];
#pragma unroll
  for (int j = 0; j < SKINNY_BATCH; ++j)
    bfv[j] = c0 + j < c1 ? *reinterpret_cast<const bf16x8_t*>(bp + (long)(c0 + j) * 32)
                         : bf16x8_t{};

  // epilogue thread: row em, columns en .. en+3
  const int em = tid / (4 * CT), en = blockIdx.x * 16 * CT + 4 * (tid % (4 * CT));
  const bool etd = tid < SKINNY_M * 4 * CT && em < M && en < N;
  float ein[4] = {0.f, 0.f, 0.f, 0.f}, eb[4];
  if (etd) {
    epi_load4<EPI, TO>(e, em, en, ein);
    epi_load_bias(e, en, eb);
  }

  if constexpr (LNA) {
    constexpr int NV = LN_SKINNY_MAX_K / 256;
    if (w < M) {
      const float* xr = x + (long)w * K;
      float4 v[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (lane * 4 + 256 * i < K) v[i] = *reinterpret_cast<const float4*>(xr + lane * 4 + 256 * i);
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (lane * 4 + 256 * i < K) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
      const float mean = wave_sum(sum) / (float)K;
      float q = 0.f;
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (lane * 4 + 256 * i < K) {
          const float d[4] = {v[i].x - mean, v[i].y - mean, v[i].z - mean, v[i].w - mean};
#pragma unroll
          for (int j = 0; j < 4; ++j) q += d[j] * d[j];
        }
      const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)K + 1e-5f);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c = lane * 4 + 256 * i;
        if (c < K) {
          const float4 g = *reinterpret_cast<const float4*>(lnw + c);
          const float4 bb = *reinterpret_cast<const float4*>(lnb + c);
          const float o0 = (v[i].x - mean) * rstd * g.x + bb.x;
          const float o1 = (v[i].y - mean) * rstd * g.y + bb.y;
          const float o2 = (v[i].z - mean) * rstd * g.z + bb.z;
          const float o3 = (v[i].w - mean) * rstd * g.w + bb.w;
          *reinterpret_cast<uint2*>(sA + (long)w * K + c) = make_uint2(pack_bf2(o0, o1),
                                                                       pack_bf2(o2, o3));
        }
      }
    }
    __syncthreads();
  }
  const bf16_t* ap = LNA ? sA + (long)(arow ? r : 0) * K + kq : A + (long)(arow ? r : 0) * lda + kq;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int cb = c0; cb < c1; cb += SKINNY_BATCH) {
    bf16x8_t af[SKINNY_BATCH];
#pragma unroll
    for (int j = 0; j < SKINNY_BATCH; ++j)
      af[j] = arow && cb + j < c1 ? *reinterpret_cast<const bf16x8_t*>(ap + (long)(cb + j) * 32)
                                  : bf16x8_t{};
#pragma unroll
    for (int j = 0; j < SKINNY_BATCH; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], bfv[j], acc, 0, 0, 0);
    // the next batch of B (a contraction of more than 8 chunks per wavefront)
#pragma unroll
    for (int j = 0; j < SKINNY_BATCH; ++j)
      bfv[j] = cb + SKINNY_BATCH + j < c1
                   ? *reinterpret_cast<const bf16x8_t*>(bp + (long)(cb + SKINNY_BATCH + j) * 32)
                   : bf16x8_t{};
  }
  // lane l holds rows 4(l/16) .. +3 of column l%16
#pragma unroll
  for (int i = 0; i < 4; ++i) red[w][(4 * (lane >> 4) + i) * 16 + r] = acc[i];
  __syncthreads();
  if (etd) {
    const int cl = en - blockIdx.x * 16 * CT, t = cl >> 4, cc = cl & 15;
    float c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a = red[t][em * 16 + cc + j];
      for (int q = 1; q < NKS; ++q) a += red[q * CT + t][em * 16 + cc + j];
      c[j] = a;
    }
    epi_store4<EPI, TO>(e, em, en, c, ein, eb, 0);
  }
}

// Whether the few-rows kernel takes this product (bf16, C = A B^T with both
// operands k-contiguous, M <= 16, K a multiple of 32, an elementwise epilogue).
bool skinny_ok(DType in_t, int M, int K, bool a_t, bool b_t, int epi) {
  return in_t == DT_BF16 && !a_t && !b_t && M >= 1 && M <= SKINNY_M && K % 32 == 0 &&
         (epi == EPI_STORE || epi == EPI_BIAS || epi == EPI_BIAS_GELU || epi == EPI_RESID ||
          epi == EPI_ACCUM);
}

template <bool LNA, int CT>
static hipError_t skinny_by_epi(int M, int N, int K, const bf16_t* A, long lda, const bf16_t* B,
                                long ldb, int epi, DType out_t, const EpiArgs& e, const float* x,
                                const float* lnw, const float* lnb, hipStream_t s) {
  const unsigned grid = (unsigned)((N + 16 * CT - 1) / (16 * CT));
  const int nt = SKINNY_WAVES * 64;
  const size_t lds = LNA ? (size_t)M * K * sizeof(bf16_t) : 0;
#define SKINNY_RUN(E, T) \
  gemm_skinny_kernel<E, T, LNA, CT><<<grid, nt, lds, s>>>(M, N, K, A, lda, B, ldb, e, x, lnw, lnb)
  switch (epi) {
    case EPI_STORE:
      if (out_t == DT_BF16) SKINNY_RUN(EPI_STORE, bf16_t);
      else SKINNY_RUN(EPI_STORE, float);
      break;
    case EPI_BIAS:
      if (out_t == DT_BF16) SKINNY_RUN(EPI_BIAS, bf16_t);
      else SKINNY_RUN(EPI_BIAS, float);
      break;
    case EPI_BIAS_GELU:
      if (out_t == DT_BF16) SKINNY_RUN(EPI_BIAS_GELU, bf16_t);
      else SKINNY_RUN(EPI_BIAS_GELU, float);
      break;
    case EPI_RESID:
      SKINNY_RUN(EPI_RESID, float);
      break;
    case EPI_ACCUM:
      SKINNY_RUN(EPI_ACCUM, float);
      break;
    default:
      return hipErrorInvalidValue;
  }
#undef SKINNY_RUN
  return hipGetLastError();
}

// Four column tiles per workgroup once there are enough columns for 512 such
// workgroups (the vocabulary-wide head), one otherwise.
constexpr int SKINNY_WIDE_N = 16 * 4 * 512;

hipError_t launch_gemm_skinny(int M, int N, int K, const bf16_t* A, long lda, const bf16_t* B,
                              long ldb, int epi, DType out_t, const EpiArgs& e, hipStream_t s) {
  if (N >= SKINNY_WIDE_N)
    return skinny_by_epi<false, 4>(M, N, K, A, lda, B, ldb, epi, out_t, e, nullptr, nullptr,
                                   nullptr, s);
  return skinny_by_epi<false, 1>(M, N, K, A, lda, B, ldb, epi, out_t, e, nullptr, nullptr,
                                 nullptr, s);
}

hipError_t launch_gemm_ln_skinny(int M, int N, int K, const float* x, const float* lnw,
                                 const float* lnb, const void* B, long ldb, int epi, DType out_t,
                                 const EpiArgs& e, hipStream_t s) {
  if (M < 1 || M > SKINNY_M || K % 32 || K > LN_SKINNY_MAX_K || ldb % 8 || N % 8)
    return hipErrorInvalidValue;
  if (N >= SKINNY_WIDE_N)
    return skinny_by_epi<true, 4>(M, N, K, nullptr, 0, (const bf16_t*)B, ldb, epi, out_t, e, x,
                                  lnw, lnb, s);
  return skinny_by_epi<true, 1>(M, N, K, nullptr, 0, (const bf16_t*)B, ldb, epi, out_t, e, x, lnw,
                                lnb, s);
}

hipError_t launch_gemm_fill(DType in_t, int M, int N, int K, const void* A, long lda, bool a_t,
                            const void* B, long ldb, bool b_t, int epi, DType out_t,
                            const EpiArgs& e, float* part, long part_elems, hipStream_t s) {
  // Too few 256-row tiles to fill the persistent grid (a few hundred rows: the
  // sampling loop's forward passes) and a deep enough contraction: K-slices
  // into fp32 scratch, then the epilogue over their sum.
  const bool kinds = epi == EPI_STORE || epi == EPI_BIAS || epi == EPI_BIAS_GELU || epi == EPI_RESID;
  if (skinny_ok(in_t, M, K, a_t, b_t, epi))
    return launch_gemm(in_t, M, N, K, A, lda, a_t, B, ldb, b_t, epi, out_t, e, 1, s);
  if (in_t == DT_BF16 && kinds && part && K % 64 == 0 && N % 4 == 0) {
    const long slots = gemm_slots();
    const long tiles = (long)((M + 255) / 256) * ((N + 255) / 256);
    const int nkt = K / 64;
    int S = (int)(slots / tiles);
    if (S > nkt / 4) S = nkt / 4;
    if (tiles * 2 <= slots && S >= 2) {
      S = exact_splits(in_t, K, S);
      while (S > 1 && (long)S * M * N > part_elems) S = exact_splits(in_t, K, S - 1);
      if (S > 1) {
        EpiArgs ep;
        memset(&ep, 0, sizeof(ep));
        ep.out = part;
        ep.ldo = N;
        ep.alpha = 1.f;
        ep.split_stride = (long)M * N;
        hipError_t r = launch_gemm(in_t, M, N, K, A, lda, a_t, B, ldb, b_t, EPI_PARTIAL, DT_F32,
                                   ep, S, s);
        if (r != hipSuccess) return r;
        const long groups = (long)M * (N / 4);
        const unsigned blocks = (unsigned)((groups + 255) / 256);
        switch (epi) {
          case EPI_STORE:
            if (out_t == DT_BF16)
              splitk_epi_kernel<EPI_STORE, bf16_t><<<blocks, 256, 0, s>>>(part, S, M, N, e);
            else
              splitk_epi_kernel<EPI_STORE, float><<<blocks, 256, 0, s>>>(part, S, M, N, e);
            break;
          case EPI_BIAS:
            splitk_epi_kernel<EPI_BIAS, bf16_t><<<blocks, 256, 0, s>>>(part, S, M, N, e);
            break;
          case EPI_BIAS_GELU:
            splitk_epi_kernel<EPI_BIAS_GELU, bf16_t><<<blocks, 256, 0, s>>>(part, S, M, N, e);
            break;
          default:
            splitk_epi_kernel<EPI_RESID, float><<<blocks, 256, 0, s>>>(part, S, M, N, e);
            break;
        }
        return hipGetLastError();
      }
    }
  }
  return launch_gemm(in_t, M, N, K, A, lda, a_t, B, ldb, b_t, epi, out_t, e, 0, s);
}

hipError_t launch_gemm(DType in_t, int M, int N, int K, const void* A, long lda, bool a_t,
                       const void* B, long ldb, bool b_t, int epi, DType out_t, const EpiArgs& e,
                       int split_k, hipStream_t s) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  if (N % 4) return hipErrorInvalidValue;
  if (in_t == DT_F32) {
    if (out_t != DT_F32) return hipErrorInvalidValue;
    const float* a = (const float*)A;
    const float* b = (const float*)B;
    if (!a_t && !b_t) return f32_by_epi<false, false>(M, N, K, a, lda, b, ldb, epi, e, split_k, s);
    if (!a_t && b_t) return f32_by_epi<false, true>(M, N, K, a, lda, b, ldb, epi, e, split_k, s);
    if (a_t && b_t) return f32_by_epi<true, true>(M, N, K, a, lda, b, ldb, epi, e, split_k, s);
    return f32_by_epi<true, false>(M, N, K, a, lda, b, ldb, epi, e, split_k, s);
  }
  // bf16: 16-byte chunks along the contiguous dimension of each operand, and
  // the epilogue writes 8 consecutive columns per lane
  if (lda % 8 || ldb % 8 || N % 8) return hipErrorInvalidValue;
  if ((!a_t || !b_t) && K % 8) return hipErrorInvalidValue;
  if ((a_t && M % 8) || (b_t && N % 8)) return hipErrorInvalidValue;
  const bf16_t* a = (const bf16_t*)A;
  const bf16_t* b = (const bf16_t*)B;
  if (skinny_ok(in_t, M, K, a_t, b_t, epi) && (epi != EPI_RESID || out_t == DT_F32) &&
      (epi != EPI_ACCUM || out_t == DT_F32))
    return launch_gemm_skinny(M, N, K, a, lda, b, ldb, epi, out_t, e, s);
  if (!a_t && !b_t)
    return gemm_mfma::dispatch<false, false>(M, N, K, a, lda, b, ldb, epi, out_t, e, split_k, s);
  if (!a_t && b_t)
    return gemm_mfma::dispatch<false, true>(M, N, K, a, lda, b, ldb, epi, out_t, e, split_k, s);
  if (a_t && b_t)
    return gemm_mfma::dispatch<true, true>(M, N, K, a, lda, b, ldb, epi, out_t, e, split_k, s);
  return hipErrorInvalidValue;
}
