// bf16 GEMM on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
//   C[m][n] = sum_k A(m,k) B(n,k),  then an epilogue (epilogue.h)
//
// A(m,k) is A[m*lda + k] (k contiguous) or, with AT, A[k*lda + m]; likewise B.
// The linear layers use three forms: forward y = x W^T (A, B both
// k-contiguous), input gradient dx = dy W (B transposed), weight gradient
// dW = dy^T x (both transposed).
//
// Block tile BM x BN x 64 with WM x WN wavefronts (2 x 4 or 4 x 2, and 4 x 4
// for the weight gradients); each wavefront owns a (BM/WM) x (BN/WN)
// sub-tile of 32x32 MFMA tiles.  When K is a multiple of 64 the operand
// tiles go straight from global memory to LDS (global_load_lds): a
// k-contiguous operand as [row][64 k] bf16 with the 16-byte chunk index
// XOR-swizzled by the row (conflict-free ds_read_b128 of MFMA fragments), a
// transposed one as [64 k][rows], whose fragments are gathered with LDS
// transpose reads (ds_read_b64_tr_b16).  Otherwise the tiles pass through
// registers, and a transposed operand is turned k-contiguous on the way: each
// thread loads an 8 (k) x 8 (row) block and transposes it with v_perm_b32.
// Two LDS stages: the global loads of tile k+1 are in flight while the MFMAs
// of tile k run; one barrier per k-tile.
//
// MFMA role assignment: the matrix-core "row" operand is the B tile (n) and
// the "column" operand the A tile (m), so each lane's accumulator holds four
// consecutive n of one m: the epilogue writes 4 consecutive columns per lane.
#pragma once
#include <type_traits>

#include "kernels.h"

namespace gemm_mfma {

constexpr int BK = 64;

__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row ^ (row >> 3)) & 7); }

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// R rows x 64 k, k contiguous in global memory; NT threads.  issue():
// 16-byte global loads into registers; commit(): ds_write into the stage.
template <int R, int NT>
struct LoaderK {
  static constexpr int RPP = NT / 8;  // rows per pass
  uint4 v[R / RPP];
  __device__ __forceinline__ void setup(const bf16_t*, long, long, long, int) {}
  __device__ __forceinline__ void issue(const bf16_t* __restrict__ X, long ld, long r0, long rtot,
                                        int k, int K, int tid, bf16_t*) {
    int c = tid & 7, rr = tid >> 3;
    bool kin = k + c * 8 < K;
#pragma unroll
    for (int i = 0; i < R / RPP; ++i) {
      long row = r0 + rr + RPP * i;
      if (kin && row < rtot)
        v[i] = *reinterpret_cast<const uint4*>(X + row * ld + k + c * 8);
      else
        v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void commit(bf16_t* s, int tid) const {
    int c = tid & 7, rr = tid >> 3;
#pragma unroll
    for (int i = 0; i < R / RPP; ++i) {
      int row = rr + RPP * i;
      *reinterpret_cast<uint4*>(s + row * BK + swz(row, c) * 8) = v[i];
    }
  }
};

// R rows x 64 k, k contiguous, K a multiple of 64: loaded straight into LDS
// with global_load_lds_dwordx4.  One wavefront instruction fills 1 KB of LDS
// = 8 rows; lane i lands in row i/8, physical chunk i%8, so it fetches the
// logical chunk (i%8) ^ swizzle(row).  Rows past the matrix edge re-read the
// last row (their products are never stored).
template <int R, int NT>
struct LoaderD {
  static constexpr int NW = NT / 64;
  static constexpr int PER_WAVE = R / 8 / NW;  // wavefront instructions per tile
  // Per tile (setup): each lane's byte offsets from the tile's first row, so
  // that a k-step only moves the wavefront-uniform base pointer.
  const char* base;
  uint32_t off[PER_WAVE];
  __device__ __forceinline__ void setup(const bf16_t* __restrict__ X, long ld, long r0, long rtot,
                                        int tid) {
    const int lane = tid & 63, w = tid >> 6;
    base = reinterpret_cast<const char*>(X + r0 * ld);
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int row = (w * PER_WAVE + j) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((row ^ (row >> 3)) & 7);
      const long lrow = r0 + row < rtot ? row : rtot - 1 - r0;
      off[j] = (uint32_t)((lrow * ld + c * 8) * 2);
    }
  }
  __device__ __forceinline__ void issue(const bf16_t* __restrict__, long, long, long, int k, int,
                                        int tid, bf16_t* s) {
    const int w = tid >> 6;
    const char* kb = base + 2L * k;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int rbase = (w * PER_WAVE + j) * 8;
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(kb + off[j]),
          (__attribute__((address_space(3))) void*)(s + rbase * BK), 16, 0, 0);
    }
  }
  __device__ __forceinline__ void commit(bf16_t*, int) const {}
};

// R rows x 64 k, rows contiguous in global memory (X[k*ld + row]).  Thread t
// moves a KR (k) x 8 (row) block, KR = 8R/NT: KR 16-byte loads along the
// rows, a register transpose with v_perm_b32, and 8 LDS writes of KR values.
template <int R, int NT>
struct LoaderT {
  static constexpr int RC = R / 8;        // 8-row chunks across the tile
  static constexpr int KR = 8 * R / NT;   // k rows per thread (2, 4 or 8)
  static_assert(KR == 2 || KR == 4 || KR == 8, "tile/thread combination");
  uint4 v[KR];
  __device__ __forceinline__ void setup(const bf16_t*, long, long, long, int) {}
  __device__ __forceinline__ void issue(const bf16_t* __restrict__ X, long ld, long r0, long rtot,
                                        int k, int K, int tid, bf16_t*) {
    int rc = tid % RC, kg = tid / RC;
    long col = r0 + rc * 8;
    bool cin = col < rtot;
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      int kk = k + kg * KR + j;
      if (cin && kk < K)
        v[j] = *reinterpret_cast<const uint4*>(X + (long)kk * ld + col);
      else
        v[j] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void commit(bf16_t* s, int tid) const {
    int rc = tid % RC, kg = tid / RC;
    const int kbase = kg * KR;  // first k of this thread inside the 64-deep tile
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const unsigned sel = (r & 1) ? 0x7632u : 0x5410u;
      int row = rc * 8 + r;
      bf16_t* dst = s + row * BK + swz(row, kbase >> 3) * 8 + (kbase & 7);
      if constexpr (KR == 8) {
        uint4 o;
        o.x = __byte_perm(word(v[0], r >> 1), word(v[1], r >> 1), sel);
        o.y = __byte_perm(word(v[2], r >> 1), word(v[3], r >> 1), sel);
        o.z = __byte_perm(word(v[4], r >> 1), word(v[5], r >> 1), sel);
        o.w = __byte_perm(word(v[6], r >> 1), word(v[7], r >> 1), sel);
        *reinterpret_cast<uint4*>(dst) = o;
      } else if constexpr (KR == 4) {
        uint2 o;
        o.x = __byte_perm(word(v[0], r >> 1), word(v[1], r >> 1), sel);
        o.y = __byte_perm(word(v[2], r >> 1), word(v[3], r >> 1), sel);
        *reinterpret_cast<uint2*>(dst) = o;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = __byte_perm(word(v[0], r >> 1), word(v[1], r >> 1), sel);
      }
    }
  }
};

// R rows x 64 k of a transposed operand (X[k*ld + row], rows contiguous), K a
// multiple of 64, loaded straight into LDS as [64 k][R rows] (R = 256 or 192).
// Wavefront instruction g fills bytes [1 KB g, 1 KB (g+1)) of the tile; the
// 16-byte chunk c of k-row kr is stored at chunk dt_phys(kr, c), which keeps
// the transpose reads of the fragments (4 consecutive k-rows x 64 bytes per
// half-wavefront) free of bank conflicts: for R = 256 (512-byte k-rows) chunk
// c ^ 4(kr%4); for R = 192 (384-byte k-rows, alternate rows half a bank
// window apart) a rotation by 4 chunks on k-rows 2 and 3 of every 4.
// Columns past the matrix edge re-read the last 8 (their products are never
// stored).
template <int R>
__device__ __forceinline__ int dt_phys(int kr, int c) {
  if constexpr (R == 256) {
    return c ^ (4 * (kr & 3));
  } else {
    static_assert(R == 192, "transposed direct tiles are 256 or 192 wide");
    const int p = c + 4 * ((kr >> 1) & 1);
    return p >= R / 8 ? p - R / 8 : p;
  }
}
template <int R>
__device__ __forceinline__ int dt_logical(int kr, int p) {
  if constexpr (R == 256) {
    return p ^ (4 * (kr & 3));
  } else {
    const int c = p - 4 * ((kr >> 1) & 1);
    return c < 0 ? c + R / 8 : c;
  }
}

template <int R, int NT>
struct LoaderDT {
  static constexpr int NW = NT / 64;
  static constexpr int CPR = R / 8;                 // 16-byte chunks per k-row
  static constexpr int NINST = BK * R * 2 / 1024;   // wavefront instructions per tile
  static constexpr int PER_WAVE = NINST / NW;
  static_assert(PER_WAVE * NW == NINST, "tile/thread combination");
  const char* base;
  uint32_t off[PER_WAVE];
  long ldb2;  // bytes per k-row in global memory
  __device__ __forceinline__ void setup(const bf16_t* __restrict__ X, long ld, long r0, long rtot,
                                        int tid) {
    const int lane = tid & 63, w = tid >> 6;
    base = reinterpret_cast<const char*>(X + r0);
    ldb2 = 2 * ld;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int chunk = (w * PER_WAVE + j) * 64 + lane;  // 16-byte chunk index in the tile
      const int kr = chunk / CPR;
      const int c = dt_logical<R>(kr, chunk - kr * CPR);
      long col = (long)c * 8;
      if (r0 + col + 8 > rtot) col = rtot - 8 - r0;
      off[j] = (uint32_t)((kr * ld + col) * 2);
    }
  }
  __device__ __forceinline__ void issue(const bf16_t* __restrict__, long, long, long, int k, int,
                                        int tid, bf16_t* s) {
    const int w = tid >> 6;
    const char* kb = base + ldb2 * k;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int g = w * PER_WAVE + j;
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(kb + off[j]),
          (__attribute__((address_space(3))) void*)(s + g * 512), 16, 0, 0);
    }
  }
  __device__ __forceinline__ void commit(bf16_t*, int) const {}
};

typedef short gemm_short4 __attribute__((ext_vector_type(4)));

// Fragment of a [64 k][R] tile for matrix row `row` (this lane's row) and
// contraction slots 8h + 0..7 of substep kk (h = lane/32), from two LDS
// transpose reads: in each 16-lane group, lane t addresses k-row t/4 and rows
// 4(t%4)..+3 of the matrix, and receives matrix row t of the 4 k-rows.
template <int R>
__device__ __forceinline__ bf16x8_t frag_tr(const bf16_t* s, int rbase, int kk, int lane) {
  const int g = lane >> 4, t = lane & 15;
  const int col = rbase + 16 * (g & 1) + 4 * (t & 3);
  uint32_t w[4];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int kr = 16 * kk + 8 * (g >> 1) + 4 * half + (t >> 2);
    const bf16_t* p = s + kr * R + (dt_phys<R>(kr, col >> 3) << 3) + (col & 7);
    const gemm_short4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) gemm_short4*)((__attribute__((address_space(3))) bf16_t*)p));
    const uint2 u = __builtin_bit_cast(uint2, v);
    w[2 * half] = u.x;
    w[2 * half + 1] = u.y;
  }
  return __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
}

// Operand layout: 0 k-contiguous via registers, 1 transposed via registers,
// 2 k-contiguous direct to LDS, 3 transposed direct to LDS.
template <int R, int L, int NT> struct Loader;
template <int R, int NT> struct Loader<R, 0, NT> : LoaderK<R, NT> {};
template <int R, int NT> struct Loader<R, 1, NT> : LoaderT<R, NT> {};
template <int R, int NT> struct Loader<R, 2, NT> : LoaderD<R, NT> {};
template <int R, int NT> struct Loader<R, 3, NT> : LoaderDT<R, NT> {};

// fp32 epilogue inputs loaded ahead per 32-row round: as many groups of
// eight as fit the registers beside the accumulators in every variant
constexpr int EPI_NPRE32 = 2;

// Eight consecutive elements of an epilogue input held as loaded (bf16 stays
// packed), so the load can be issued well before its values are needed.
template <typename T> struct In8;
template <> struct In8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void get(float v[8]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};
template <> struct In8<bf16_t> {
  uint4 a;
  __device__ __forceinline__ void load(const bf16_t* p) { a = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void get(float v[8]) const {
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

// Epilogue of one output tile, staged through LDS so that global memory sees
// whole row segments.  acc[sn][sm][4i + j] is C[m][n] with m = sm*32 +
// lane%32 and n = sn*32 + 8i + 4(lane/32) + j inside the wavefront's
// (BM/WM) x (BN/WN) sub-tile.  Each wavefront owns a round buffer of scratch
// LDS and moves its sub-tile in rounds of rows: (1) lanes write alpha * their
// accumulator fragments, fp32, into a row-major round buffer (16-byte chunks
// XOR-swizzled by row, so both the fragment writes and the row reads are
// bank-conflict free); (2) lanes read back 8 consecutive columns of one row
// each -- 8 lanes cover the 64 columns of a row -- apply the elementwise
// epilogue and store 16-byte pieces, so one store instruction writes 8
// complete row segments.
// Rows per epilogue round: 32, or 16 when the wavefronts' 32-row buffers
// would not fit one LDS stage (16 wavefronts on a 256 x 256 tile); a round
// buffer takes ROWS x 64 fp32 = ROWS x 128 bf16 elements of scratch.
template <int BM, int BN, int WM, int WN>
constexpr int epi_rows() {
  return (BM + BN) * BK >= WM * WN * 32 * 128 ? 32 : 16;
}

template <int BM, int BN, int WM, int WN, int EPI, typename TO, int SN, int SM>
__device__ __forceinline__ void tile_epilogue(const EpiArgs& e, const f32x16_t (&acc)[SN][SM],
                                              long m0, long n0, int split, int M, int N, int lane,
                                              int wm, int wn, bf16_t* scratch) {
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int ROWS = epi_rows<BM, BN, WM, WN>();
  static_assert(WTN == 64, "staged epilogue assumes 64-column wavefront sub-tiles");
  static_assert((BM + BN) * BK >= WM * WN * ROWS * 128, "epilogue scratch must fit one LDS stage");
  float* sf = reinterpret_cast<float*>(scratch);  // [ROWS rows][64 fp32]
  const long mw = m0 + wm * WTM;                  // first row of the sub-tile
  const long nl = n0 + wn * WTN + (lane & 7) * 8; // this lane's 8 columns in the read phase
  const bool ncol = nl < N;
  float bias8[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) bias8[j] = 0.f;
  if constexpr (epi_bias(EPI)) {
    if (e.bias && ncol) {
      ld4(e.bias + nl, bias8);
      ld4(e.bias + nl + 4, bias8 + 4);
    }
  }
  // EPI_GELU_BWD: column sums of the result over the sub-tile's rows (the
  // bias gradient of the layer that produced the pre-activation)
  float csum[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) csum[j] = 0.f;
  float dl_nv = 0.f;  // EPI_DLOGITS: 1 / n_valid
  if constexpr (EPI == EPI_DLOGITS) {
    const int nv = *e.n_valid;
    dl_nv = nv > 0 ? 1.0f / (float)nv : 0.f;
  }
#pragma unroll
  for (int sm = 0; sm < SM; ++sm) {
    // EPI_DLOGITS: target and log-sum-exp of this lane's rows of the round,
    // loaded ahead of the LDS round trip
    int dtg[4];
    float dls[4];
    if constexpr (EPI == EPI_DLOGITS) {
#pragma unroll
      for (int r8 = 0; r8 < 4; ++r8) {
        const long m = mw + sm * 32 + r8 * 8 + (lane >> 3);
        dtg[r8] = m < M ? e.tgt[m] : -1;
        dls[r8] = m < M ? e.lse[m] : 0.f;
      }
    }
    // inputs of the elementwise epilogue for the round's row groups, issued
    // before the LDS round trip so that their latencies overlap instead of
    // each group's load, wait and store running in turn: bf16 inputs for all
    // four groups, fp32 ones for the first EPI_NPRE32 (addresses clamped to
    // row M-1 and column 0 where the row or the lane's columns lie past the
    // matrix; those values are not used)
    constexpr bool PRE = EPI == EPI_RESID || EPI == EPI_ACCUM || EPI == EPI_GELU_BWD;
    using PreT = std::conditional_t<EPI == EPI_GELU_BWD, TO, float>;
    constexpr int NPRE = !PRE ? 0 : sizeof(PreT) == 2 ? 4 : EPI_NPRE32;
    [[maybe_unused]] In8<PreT> pre[4];
    if constexpr (PRE) {
#pragma unroll
      for (int r8 = 0; r8 < NPRE; ++r8) {
        const long m = mw + sm * 32 + r8 * 8 + (lane >> 3);
        const long mc = m < M ? m : M - 1;
        const long nc = ncol ? nl : 0;
        if constexpr (EPI == EPI_RESID) pre[r8].load(e.resid + mc * e.ldr + nc);
        else if constexpr (EPI == EPI_ACCUM)
          pre[r8].load(reinterpret_cast<const float*>(e.out) + mc * e.ldo + nc);
        else pre[r8].load(reinterpret_cast<const TO*>(e.aux) + mc * e.ldx + nc);
      }
    }
#pragma unroll
    for (int hr = 0; hr < 32 / ROWS; ++hr) {
    // (1) fragments -> round buffer (row = lane%32, one 16-byte chunk each;
    // with 16-row rounds, the lanes whose row lies in this round)
    if (ROWS == 32 || ((lane & 31) >> 4) == hr) {
      const int row = (lane & 31) - hr * ROWS;
#pragma unroll
      for (int sn = 0; sn < SN; ++sn)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = (sn * 32 + 8 * i + 4 * (lane >> 5)) >> 2;
          const int pc = c ^ (row & 7);
          *reinterpret_cast<float4*>(sf + row * 64 + pc * 4) =
              make_float4(e.alpha * acc[sn][sm][4 * i + 0], e.alpha * acc[sn][sm][4 * i + 1],
                          e.alpha * acc[sn][sm][4 * i + 2], e.alpha * acc[sn][sm][4 * i + 3]);
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // (2) rows of the round -> global, 8 lanes per row; r8 counts the round's
    // 8-row groups over the whole 32-row block
#pragma unroll
    for (int r8 = hr * (ROWS / 8); r8 < (hr + 1) * (ROWS / 8); ++r8) {
      const int row = r8 * 8 + (lane >> 3) - hr * ROWS;
      const long m = mw + sm * 32 + hr * ROWS + row;
      const int c0 = (2 * (lane & 7)) ^ (row & 7), c1 = (2 * (lane & 7) + 1) ^ (row & 7);
      const float4 a = *reinterpret_cast<const float4*>(sf + row * 64 + c0 * 4);
      const float4 b = *reinterpret_cast<const float4*>(sf + row * 64 + c1 * 4);
      float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      if (m < M && ncol) {
        if constexpr (epi_bias(EPI)) {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] += bias8[j];
        }
        if constexpr (EPI == EPI_STORE || EPI == EPI_BIAS) {
          st4(reinterpret_cast<TO*>(e.out) + m * e.ldo + nl, v);
          st4(reinterpret_cast<TO*>(e.out) + m * e.ldo + nl + 4, v + 4);
        } else if constexpr (EPI == EPI_DLOGITS) {
          const int t = dtg[r8];
          const float l = dls[r8], sc = t != -1 ? dl_nv : 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = dlogit(v[j], l, e.col0 + nl + j == t, sc);
          st4(reinterpret_cast<TO*>(e.out) + m * e.ldo + nl, v);
          st4(reinterpret_cast<TO*>(e.out) + m * e.ldo + nl + 4, v + 4);
        } else if constexpr (EPI == EPI_BIAS_GELU) {
          float d[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = gelu_tanh_and_grad_f(v[j], d + j);
          st4(reinterpret_cast<TO*>(e.out) + m * e.ldo + nl, d);
          st4(reinterpret_cast<TO*>(e.out) + m * e.ldo + nl + 4, d + 4);
          st4(reinterpret_cast<TO*>(e.out2) + m * e.ldo + nl, v);
          st4(reinterpret_cast<TO*>(e.out2) + m * e.ldo + nl + 4, v + 4);
        } else if constexpr (EPI == EPI_RESID) {
          float x[8];
          if (r8 < NPRE) {
            pre[r8].get(x);
          } else {
            ld4(e.resid + m * e.ldr + nl, x);
            ld4(e.resid + m * e.ldr + nl + 4, x + 4);
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] += x[j];
          st4(reinterpret_cast<float*>(e.out) + m * e.ldo + nl, v);
          st4(reinterpret_cast<float*>(e.out) + m * e.ldo + nl + 4, v + 4);
        } else if constexpr (EPI == EPI_ACCUM) {
          float* o = reinterpret_cast<float*>(e.out) + m * e.ldo + nl;
          float x[8];
          if (r8 < NPRE) {
            pre[r8].get(x);
          } else {
            ld4(o, x);
            ld4(o + 4, x + 4);
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] += x[j];
          st4(o, v);
          st4(o + 4, v + 4);
        } else if constexpr (EPI == EPI_ATOMIC) {
          float* o = reinterpret_cast<float*>(e.out) + m * e.ldo + nl;
#pragma unroll
          for (int j = 0; j < 8; ++j) atomicAdd(o + j, v[j]);
        } else if constexpr (EPI == EPI_PARTIAL) {
          float* o = reinterpret_cast<float*>(e.out) + split * e.split_stride + m * e.ldo + nl;
          st4(o, v);
          st4(o + 4, v + 4);
        } else if constexpr (EPI == EPI_GELU_BWD) {
          float dg[8];
          if (r8 < NPRE) {
            pre[r8].get(dg);
          } else {
            ld4(reinterpret_cast<const TO*>(e.aux) + m * e.ldx + nl, dg);
            ld4(reinterpret_cast<const TO*>(e.aux) + m * e.ldx + nl + 4, dg + 4);
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            v[j] *= dg[j];
            csum[j] += v[j];
          }
          st4(reinterpret_cast<TO*>(e.out) + m * e.ldo + nl, v);
          st4(reinterpret_cast<TO*>(e.out) + m * e.ldo + nl + 4, v + 4);
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (EPI == EPI_GELU_BWD) {
    if (e.colsum) {
      // lanes l, l^8, ..., l^56 hold the same 8 columns for different rows
#pragma unroll
      for (int o = 8; o < 64; o <<= 1)
#pragma unroll
        for (int j = 0; j < 8; ++j) csum[j] += __shfl_xor(csum[j], o, 64);
      static_assert(WTM == 128, "column sums are kept per 128-row block");
      // a sub-tile wholly past the last row has no block of its own: its
      // index ceil(M/128) is one past the rows the slot holds for M rows
      if (lane < 8 && ncol && mw < M) {
        float* dst = e.colsum + (mw / 128) * (long)N + nl;
        st4(dst, csum);
        st4(dst + 4, csum + 4);
      }
    }
  }
}

// EPI_LSE straight from the accumulators, no LDS staging: for each of its
// rows a lane holds 32 of the wavefront's 64 columns (col = sn*32 + 8i + 4h +
// j, h = lane/32) and lane ^ 32 the other 32, so a row's block maximum and
// sum of exponentials take 32 lane-local steps and one exchange.  (alpha is
// not applied: the logits are the plain products.)
template <int BM, int BN, int WM, int WN, int SN, int SM>
__device__ __forceinline__ void lse_epilogue(const EpiArgs& e, const f32x16_t (&acc)[SN][SM],
                                             long m0, long n0, int M, int N, int lane, int wm,
                                             int wn) {
  constexpr int WTM = BM / WM, WTN = BN / WN;
  static_assert(WTN == 64 && SN == 2, "one 64-column block of the row partials per wavefront");
  const long mw = m0 + wm * WTM, nw = n0 + wn * WTN;
  if (nw >= N) return;  // the whole block lies past the last column
  // valid columns of the block, a multiple of 8, so a lane's group of 4
  // columns is valid or not as a whole
  const int lim = N - nw < 64 ? (int)(N - nw) : 64;
  const int h4 = 4 * (lane >> 5);
  float2* part = reinterpret_cast<float2*>(e.part) + nw / 64;
#pragma unroll
  for (int sm = 0; sm < SM; ++sm) {
    const long m = mw + sm * 32 + (lane & 31);
    const bool mrow = m < M;
    const int t = mrow ? e.tgt[m] : -1;
    float mx = -__builtin_inff();
#pragma unroll
    for (int g = 0; g < 8; ++g) {  // g = sn*4 + i: columns 8g + h4 .. 8g + h4 + 3
      if (8 * g + h4 < lim) {
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, acc[g >> 2][sm][4 * (g & 3) + j]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float sum = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if (8 * g + h4 < lim) {
#pragma unroll
        for (int j = 0; j < 4; ++j) sum += __expf(acc[g >> 2][sm][4 * (g & 3) + j] - mx);
      }
    }
    sum += __shfl_xor(sum, 32, 64);
    if (mrow) {
      if (h4 == 0) part[m * e.nblk] = make_float2(mx, sum);
      const long c = (long)t - e.col0 - nw;  // the target's column within the block
      if (c >= 0 && c < lim && (int)(c & 4) == h4) {
        const int cg = (int)(c >> 3), cj = (int)(c & 3);
        float tl = 0.f;
#pragma unroll
        for (int g = 0; g < 8; ++g)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (g == cg && j == cj) tl = acc[g >> 2][sm][4 * (g & 3) + j];
        e.tlogit[m] = tl;
      }
    }
  }
}

// The same staged epilogue for 64 x 96 wavefront sub-tiles (the 256 x 192
// tile): rounds of 16 rows x 96 fp32, rows padded to 100 fp32 (400 bytes,
// 6.25 KB of scratch per wavefront), which spreads both the fragment writes
// (16 rows at one chunk) and the row reads over all banks.  In the read
// phase the round's 16 x 12 groups of 8 columns are spread over the lanes,
// three per lane.
template <int BM, int BN, int WM, int WN, int EPI, typename TO, int SN, int SM>
__device__ __forceinline__ void tile_epilogue_w96(const EpiArgs& e, const f32x16_t (&acc)[SN][SM],
                                                  long m0, long n0, int split, int M, int N,
                                                  int lane, int wm, int wn, bf16_t* scratch) {
  constexpr int WTM = BM / WM, WTN = BN / WN;
  static_assert(WTN == 96 && SN == 3, "64 x 96 wavefront sub-tiles");
  static_assert(EPI != EPI_GELU_BWD, "column sums are produced by the 64-column epilogue only");
  static_assert((BM + BN) * BK >= WM * WN * 3200, "epilogue scratch must fit one LDS stage");
  constexpr int RS = WTN + 4;  // padded round-row stride (fp32)
  float* sf = reinterpret_cast<float*>(scratch);  // [16 rows][RS fp32]
  const long mw = m0 + wm * WTM;
  const long nw = n0 + wn * WTN;
  // this lane's three (row, 8-column group) items of every round
  int irow[3], icol[3];
  float bias[3][8];
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const int p = lane + 64 * t;
    irow[t] = p / 12;
    icol[t] = (p % 12) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) bias[t][j] = 0.f;
    if constexpr (epi_bias(EPI)) {
      if (e.bias && nw + icol[t] < N) {
        ld4(e.bias + nw + icol[t], bias[t]);
        ld4(e.bias + nw + icol[t] + 4, bias[t] + 4);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < WTM / 16; ++q) {
    const int sm = q >> 1;
    // (1) fragments of rows 16q .. 16q+15 -> round buffer
    if (((lane & 31) >> 4) == (q & 1)) {
      const int row = lane & 15;
#pragma unroll
      for (int sn = 0; sn < SN; ++sn)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = sn * 8 + 2 * i + (lane >> 5);
          *reinterpret_cast<float4*>(sf + row * RS + c * 4) =
              make_float4(e.alpha * acc[sn][sm][4 * i + 0], e.alpha * acc[sn][sm][4 * i + 1],
                          e.alpha * acc[sn][sm][4 * i + 2], e.alpha * acc[sn][sm][4 * i + 3]);
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // (2) rows of the round -> global
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int row = irow[t];
      const long m = mw + q * 16 + row;
      const long n = nw + icol[t];
      const float4 a = *reinterpret_cast<const float4*>(sf + row * RS + icol[t]);
      const float4 b = *reinterpret_cast<const float4*>(sf + row * RS + icol[t] + 4);
      float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      if (m < M && n < N) {
        if constexpr (epi_bias(EPI)) {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] += bias[t][j];
        }
        if constexpr (EPI == EPI_STORE || EPI == EPI_BIAS) {
          st4(reinterpret_cast<TO*>(e.out) + m * e.ldo + n, v);
          st4(reinterpret_cast<TO*>(e.out) + m * e.ldo + n + 4, v + 4);
        } else if constexpr (EPI == EPI_BIAS_GELU) {
          float d[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = gelu_tanh_and_grad_f(v[j], d + j);
          st4(reinterpret_cast<TO*>(e.out) + m * e.ldo + n, d);
          st4(reinterpret_cast<TO*>(e.out) + m * e.ldo + n + 4, d + 4);
          st4(reinterpret_cast<TO*>(e.out2) + m * e.ldo + n, v);
          st4(reinterpret_cast<TO*>(e.out2) + m * e.ldo + n + 4, v + 4);
        } else if constexpr (EPI == EPI_RESID) {
          float x[8];
          ld4(e.resid + m * e.ldr + n, x);
          ld4(e.resid + m * e.ldr + n + 4, x + 4);
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] += x[j];
          st4(reinterpret_cast<float*>(e.out) + m * e.ldo + n, v);
          st4(reinterpret_cast<float*>(e.out) + m * e.ldo + n + 4, v + 4);
        } else if constexpr (EPI == EPI_ACCUM) {
          float* o = reinterpret_cast<float*>(e.out) + m * e.ldo + n;
          float x[8];
          ld4(o, x);
          ld4(o + 4, x + 4);
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] += x[j];
          st4(o, v);
          st4(o + 4, v + 4);
        } else if constexpr (EPI == EPI_ATOMIC) {
          float* o = reinterpret_cast<float*>(e.out) + m * e.ldo + n;
#pragma unroll
          for (int j = 0; j < 8; ++j) atomicAdd(o + j, v[j]);
        } else if constexpr (EPI == EPI_PARTIAL) {
          float* o = reinterpret_cast<float*>(e.out) + split * e.split_stride + m * e.ldo + n;
          st4(o, v);
          st4(o + 4, v + 4);
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }
}

// WM x WN wavefronts; each owns a (BM/WM) x (BN/WN) sub-tile.  Persistent:
// the grid is about one workgroup per CU; each walks the work items
// (tile, k-slice) blockIdx.x, +gridDim.x, ...
//
// GRP: a group of independent products sharing K, one persistent launch over
// the tiles of all of them (no k-slices): tile t belongs to the problem p
// with probs[p].item0 <= t < probs[p+1].item0; the kernel's M, N, A, B and
// the epilogue's out, ldo, alpha come from that problem (the tiles_m x
// tiles_n arguments are then the total tile count x 1).  Direct loaders only.
template <int BM, int BN, int WM, int WN, int LA, int LB, int EPI, typename TO, bool GRP = false>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_kernel(int M, int N, int K,
                                                      const bf16_t* __restrict__ A, long lda,
                                                      const bf16_t* __restrict__ B, long ldb,
                                                      EpiArgs e, int tiles_m, int tiles_n,
                                                      int kt_per_split,
                                                      const GemmProblem* __restrict__ probs,
                                                      int nprobs) {
  static_assert(!GRP || (LA >= 2 && LB >= 2 && BM == 256 && BN == 256),
                "grouped products use the direct loaders and 256 x 256 tiles");
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int SM = WTM / 32, SN = WTN / 32;
  // Where a k-step issues the loads of the next k-tile: right after its
  // barrier, or -- with a transposed operand, whose fragment reads are the
  // heavier -- once the fragments of its first two substeps are read, so
  // that those reads do not queue behind the loads' address traffic.  (On
  // the measured shapes each placement was the faster for its layout.)
  constexpr bool issue_late = LA == 3 || LB == 3;
  __shared__ __attribute__((aligned(16))) bf16_t smem[2][(BM + BN) * BK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;

  // Tile order: item i runs on XCD i % 8 (the grid is a multiple of 8), so
  // each XCD is given a contiguous range of tile ids -- tiles sharing operand
  // rows share that XCD's L2 -- walked in groups of 8 M-tiles.
  const int ntiles = tiles_m * tiles_n;
  const int nkt = (K + BK - 1) / BK;
  const int nsplit = (nkt + kt_per_split - 1) / kt_per_split;
  const long nitems = (long)ntiles * nsplit;
  long m0 = 0, n0 = 0;
  int kt0 = 0, kt1 = 0, split = 0;
  int prob = 0;  // GRP: the problem of the decoded item
  auto decode = [&](long it) {
    split = (int)(it / ntiles);
    int pid = (int)(it - (long)split * ntiles);
    {
      int q = ntiles >> 3, r = ntiles & 7, x = pid & 7, loc = pid >> 3;
      pid = x * q + (x < r ? x : r) + loc;
    }
    int tm = tiles_m, tn = tiles_n;
    if constexpr (GRP) {
      int lo = 0, hi = nprobs - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (probs[mid].item0 <= pid) lo = mid;
        else hi = mid - 1;
      }
      prob = lo;
      pid -= (int)probs[lo].item0;
      tm = probs[lo].tiles_m;
      tn = probs[lo].tiles_n;
    }
    constexpr int GROUP = 8;
    const int per_group = GROUP * tn;
    const int first_m = (pid / per_group) * GROUP;
    const int gsize = (tm - first_m) < GROUP ? (tm - first_m) : GROUP;
    m0 = (long)(first_m + (pid % per_group) % gsize) * BM;
    n0 = (long)((pid % per_group) / gsize) * BN;
    kt0 = split * kt_per_split;
    kt1 = (kt0 + kt_per_split) < nkt ? (kt0 + kt_per_split) : nkt;
  };
  // operands of the decoded item's problem
  auto setup = [&](auto& la_, auto& lb_) {
    if constexpr (GRP) {
      const GemmProblem& P = probs[prob];
      la_.setup(P.A, P.lda, m0, P.M, tid);
      lb_.setup(P.B, P.ldb, n0, P.N, tid);
    } else {
      la_.setup(A, lda, m0, M, tid);
      lb_.setup(B, ldb, n0, N, tid);
    }
  };
  long item = blockIdx.x;
  if (item >= nitems) return;
  decode(item);

  f32x16_t acc[SN][SM];
  Loader<BM, LA, NT> la;
  Loader<BN, LB, NT> lb;
  setup(la, lb);
  la.issue(A, lda, m0, M, kt0 * BK, K, tid, smem[0]);
  lb.issue(B, ldb, n0, N, kt0 * BK, K, tid, smem[0] + BM * BK);
  la.commit(smem[0], tid);
  lb.commit(smem[0] + BM * BK, tid);

  // Fragments of k-substep kk (16 deep) for this wavefront's sub-tiles.
  auto load_frags = [&](const bf16_t* sA, const bf16_t* sB, int kk, bf16x8_t* fa, bf16x8_t* fb) {
    const int c = kk * 2 + (lane >> 5);
#pragma unroll
    for (int sm = 0; sm < SM; ++sm) {
      if constexpr (LA == 3) {
        fa[sm] = frag_tr<BM>(sA, wm * WTM + sm * 32, kk, lane);
      } else {
        int row = wm * WTM + sm * 32 + (lane & 31);
        fa[sm] = *reinterpret_cast<const bf16x8_t*>(sA + row * BK + swz(row, c) * 8);
      }
    }
#pragma unroll
    for (int sn = 0; sn < SN; ++sn) {
      if constexpr (LB == 3) {
        fb[sn] = frag_tr<BN>(sB, wn * WTN + sn * 32, kk, lane);
      } else {
        int row = wn * WTN + sn * 32 + (lane & 31);
        fb[sn] = *reinterpret_cast<const bf16x8_t*>(sB + row * BK + swz(row, c) * 8);
      }
    }
  };

  // Software pipeline: each k-step starts by waiting for its k-tile and a
  // barrier; the loads of the next k-tile -- of this item, or the first
  // k-tile of the next item -- go out at the start of the k-step and are in
  // flight during the rest of it; the LDS fragments of substep kk+1 are
  // read while the MFMAs of substep kk run.  The epilogue's stores overlap
  // the next item's first k-step.
  bf16x8_t fa[2][SM], fb[2][SN];
  int cur = 0;
  while (true) {
#pragma unroll
    for (int a = 0; a < SN; ++a)
#pragma unroll
      for (int b = 0; b < SM; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
    const long em0 = m0, en0 = n0;  // this item's output tile
    const int ekt1 = kt1, esplit = split, eprob = prob;
    for (int kt = kt0; kt < ekt1; ++kt) {
      const bool last_k = kt + 1 == ekt1;
      const bool more = !last_k || item + gridDim.x < nitems;
      // (the first k-tile of a later item was waited for before the previous
      // epilogue, whose stores then drain during this k-step)
      if constexpr (LA >= 2 || LB >= 2)
        if (kt != kt0 || item == blockIdx.x) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // this k-tile is in LDS; the other stage is free
      const bf16_t* sA = smem[cur];
      const bf16_t* sB = smem[cur] + BM * BK;
      auto issue_next = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        if (more) {
          if (last_k) {
            decode(item + gridDim.x);
            setup(la, lb);
          }
          const int nk = last_k ? kt0 : kt + 1;
          la.issue(A, lda, m0, M, nk * BK, K, tid, smem[cur ^ 1]);
          lb.issue(B, ldb, n0, N, nk * BK, K, tid, smem[cur ^ 1] + BM * BK);
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      auto mfmas = [&](int j) {
#pragma unroll
        for (int sn = 0; sn < SN; ++sn)
#pragma unroll
          for (int sm = 0; sm < SM; ++sm)
            acc[sn][sm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j][sn], fa[j][sm], acc[sn][sm],
                                                                  0, 0, 0);
      };
      if constexpr (!issue_late) issue_next();
      load_frags(sA, sB, 0, fa[0], fb[0]);
      load_frags(sA, sB, 1, fa[1], fb[1]);
      if constexpr (issue_late) issue_next();
      mfmas(0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 1; kk < BK / 16; ++kk) {
        if (kk + 1 < BK / 16) load_frags(sA, sB, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
        mfmas(kk & 1);
        // keep the two-deep fragment pipeline: nothing moves across substeps
        __builtin_amdgcn_sched_barrier(0);
      }
      if (more) {
        la.commit(smem[cur ^ 1], tid);
        lb.commit(smem[cur ^ 1] + BM * BK, tid);
      }
      cur ^= 1;
    }
    if constexpr (LA >= 2 || LB >= 2) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // the last k-tile's stage is free; the next k-tile is in LDS
    // the stage not holding the next item's first k-tile is free: one
    // epilogue round buffer per wavefront (epi_rows x 256 bytes)
    if constexpr (GRP) {
      const GemmProblem& P = probs[eprob];
      EpiArgs eg = e;
      eg.out = P.out;
      eg.ldo = P.ldo;
      eg.alpha = P.scaled ? P.alpha * e.alpha : P.alpha;
      tile_epilogue<BM, BN, WM, WN, EPI, TO, SN, SM>(
          eg, acc, em0, en0, esplit, P.M, P.N, lane, wm, wn,
          smem[cur ^ 1] + wave * (epi_rows<BM, BN, WM, WN>() * 128));
    } else if constexpr (EPI == EPI_LSE)
      lse_epilogue<BM, BN, WM, WN, SN, SM>(e, acc, em0, en0, M, N, lane, wm, wn);
    else if constexpr (WTN == 64)
      tile_epilogue<BM, BN, WM, WN, EPI, TO, SN, SM>(
          e, acc, em0, en0, esplit, M, N, lane, wm, wn,
          smem[cur ^ 1] + wave * (epi_rows<BM, BN, WM, WN>() * 128));
    else
      tile_epilogue_w96<BM, BN, WM, WN, EPI, TO, SN, SM>(e, acc, em0, en0, esplit, M, N, lane, wm,
                                                         wn, smem[cur ^ 1] + wave * 3200);
    item += gridDim.x;
    // (the next k-step's barrier orders the scratch reads before the loads
    // that land in this stage)
    if (item >= nitems) break;
  }
}

// Host side: launch one instantiation.
// Workgroups resident at once: one per CU (the 256 x 256 tile uses 128 KB of
// LDS); rounded to a multiple of the 8 XCDs.
inline int persistent_slots() {
  static int slots = 0;
  if (!slots) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    slots = (cus + 7) / 8 * 8;
  }
  return slots;
}

template <int BM, int BN, int WM, int WN, int LA, int LB, int EPI, typename TO>
hipError_t run(int M, int N, int K, const bf16_t* A, long lda, const bf16_t* B, long ldb,
               const EpiArgs& e, int split_k, hipStream_t s) {
  int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int nkt = (K + BK - 1) / BK;
  if (split_k < 1) split_k = 1;
  int kps = (nkt + split_k - 1) / split_k;
  int splits = (nkt + kps - 1) / kps;
  long items = (long)tiles_m * tiles_n * splits;
  long grid = items < persistent_slots() ? items : persistent_slots();
  gemm_kernel<BM, BN, WM, WN, LA, LB, EPI, TO><<<(unsigned)grid, 64 * WM * WN, 0, s>>>(
      M, N, K, A, lda, B, ldb, e, tiles_m, tiles_n, kps, nullptr, 0);
  return hipGetLastError();
}

// A group of products out_p += alpha_p A_p(m,k) B_p(n,k), both operands
// transposed (k-major in memory, the weight-gradient form), all with the
// same K (a multiple of 64), in one persistent launch over total_tiles
// 256 x 256 tiles.  d_probs: nprobs device descriptors, item0 ascending from 0.
// store: out_p = instead of out_p +=.
inline hipError_t run_grouped_accum_tt(const GemmProblem* d_probs, int nprobs, long total_tiles,
                                       int K, float scale, bool store, hipStream_t s) {
  if (K % BK || total_tiles <= 0 || nprobs <= 0) return hipErrorInvalidValue;
  EpiArgs e{};
  e.alpha = scale;
  const int nkt = K / BK;
  long grid = total_tiles < persistent_slots() ? total_tiles : persistent_slots();
  if (store)
    gemm_kernel<256, 256, 4, 4, 3, 3, EPI_STORE, float, true><<<(unsigned)grid, 1024, 0, s>>>(
        0, 0, K, nullptr, 0, nullptr, 0, e, (int)total_tiles, 1, nkt, d_probs, nprobs);
  else
    gemm_kernel<256, 256, 4, 4, 3, 3, EPI_ACCUM, float, true><<<(unsigned)grid, 1024, 0, s>>>(
        0, 0, K, nullptr, 0, nullptr, 0, e, (int)total_tiles, 1, nkt, d_probs, nprobs);
  return hipGetLastError();
}

// Tile-shape choice and epilogue dispatch for one operand layout.
template <bool AT, bool BT>
hipError_t dispatch(int M, int N, int K, const bf16_t* A, long lda, const bf16_t* B, long ldb,
                    int epi, DType out_t, const EpiArgs& e, int split_k, hipStream_t s);

}  // namespace gemm_mfma

// Explicit instantiation of the epilogues of one operand layout.  Tile
// shapes: 256 x 256 x 64 with 8 wavefronts (2 x 4, each 128 x 64), and for
// outputs whose width is a multiple of 192 -- where it keeps more CUs busy --
// 256 x 192 x 64 with 8 wavefronts (4 x 2, each 64 x 96; direct loads only,
// no atomic, column-sum or fused-head epilogues).
#define GEMM_MFMA_DEFINE_DISPATCH(AT, BT)                                                       \
  namespace gemm_mfma {                                                                         \
  template <int BN_, int WM_, int WN_, int LA, int LB>                                         \
  static hipError_t by_epi(int M, int N, int K, const bf16_t* A, long lda, const bf16_t* B,    \
                           long ldb, int epi, DType out_t, const EpiArgs& e, int sk,            \
                           hipStream_t s) {                                                     \
    switch (epi) {                                                                              \
      case EPI_STORE:                                                                           \
        return out_t == DT_BF16                                                                 \
                   ? run<256, BN_, WM_, WN_, LA, LB, EPI_STORE, bf16_t>(M, N, K, A, lda, B, ldb, e, 1, s) \
                   : run<256, BN_, WM_, WN_, LA, LB, EPI_STORE, float>(M, N, K, A, lda, B, ldb, e, 1, s); \
      case EPI_BIAS:                                                                            \
        if (out_t != DT_BF16) return hipErrorInvalidValue;                                      \
        return run<256, BN_, WM_, WN_, LA, LB, EPI_BIAS, bf16_t>(M, N, K, A, lda, B, ldb, e, 1, s); \
      case EPI_BIAS_GELU:                                                                       \
        return run<256, BN_, WM_, WN_, LA, LB, EPI_BIAS_GELU, bf16_t>(M, N, K, A, lda, B, ldb, e, 1, s); \
      case EPI_RESID:                                                                           \
        return run<256, BN_, WM_, WN_, LA, LB, EPI_RESID, float>(M, N, K, A, lda, B, ldb, e, 1, s); \
      case EPI_ACCUM:                                                                           \
        return run<256, BN_, WM_, WN_, LA, LB, EPI_ACCUM, float>(M, N, K, A, lda, B, ldb, e, 1, s); \
      case EPI_ATOMIC:                                                                          \
        if constexpr (BN_ == 256)                                                               \
          return run<256, 256, 2, 4, LA, LB, EPI_ATOMIC, float>(M, N, K, A, lda, B, ldb, e, sk, s); \
        break;                                                                                  \
      case EPI_GELU_BWD:                                                                        \
        if constexpr (BN_ == 256)                                                               \
          return run<256, 256, 2, 4, LA, LB, EPI_GELU_BWD, bf16_t>(M, N, K, A, lda, B, ldb, e, 1, s); \
        break;                                                                                  \
      case EPI_PARTIAL:                                                                         \
        return run<256, BN_, WM_, WN_, LA, LB, EPI_PARTIAL, float>(M, N, K, A, lda, B, ldb, e, sk, s); \
      /* fused lm_head: logits = x wte^T only (neither operand transposed) */                    \
      case EPI_LSE:                                                                             \
        if constexpr (BN_ == 256 && LA % 2 == 0 && LB % 2 == 0)                                 \
          return run<256, 256, 2, 4, LA, LB, EPI_LSE, float>(M, N, K, A, lda, B, ldb, e, 1, s); \
        break;                                                                                  \
      case EPI_DLOGITS:                                                                         \
        if constexpr (BN_ == 256 && LA % 2 == 0 && LB % 2 == 0)                                 \
          return run<256, 256, 2, 4, LA, LB, EPI_DLOGITS, bf16_t>(M, N, K, A, lda, B, ldb, e, 1, s); \
        break;                                                                                  \
    }                                                                                           \
    return hipErrorInvalidValue;                                                                \
  }                                                                                             \
  /* fraction of the persistent workgroup slots busy over the rounds of tiles */               \
  static double slot_use(long tiles) {                                                         \
    const long slots = persistent_slots();                                                     \
    const long rounds = (tiles + slots - 1) / slots;                                           \
    return (double)tiles / (double)(rounds * slots);                                           \
  }                                                                                             \
  template <>                                                                                   \
  hipError_t dispatch<AT, BT>(int M, int N, int K, const bf16_t* A, long lda, const bf16_t* B,  \
                              long ldb, int epi, DType out_t, const EpiArgs& e, int split_k,    \
                              hipStream_t s) {                                                  \
    if (epi == EPI_ATOMIC && split_k == 0) {                                                    \
      long tiles = (long)((M + 255) / 256) * ((N + 255) / 256);                                 \
      int nkt = (K + BK - 1) / BK;                                                              \
      long want = (512 + tiles - 1) / tiles;                                                    \
      long cap = nkt / 4 > 0 ? nkt / 4 : 1;                                                     \
      split_k = (int)(want < cap ? want : cap);                                                 \
    }                                                                                           \
    /* operands go straight to LDS when whole 64-deep tiles exist */                            \
    const bool direct = K % 64 == 0;                                                            \
    constexpr int TA = AT ? 1 : 0, TB = BT ? 1 : 0;                                             \
    if (direct) {                                                                               \
      const bool w192 = N % 192 == 0 && !e.colsum &&                                            \
                        (epi == EPI_STORE || epi == EPI_BIAS || epi == EPI_BIAS_GELU ||         \
                         epi == EPI_RESID || epi == EPI_ACCUM || epi == EPI_PARTIAL);           \
      /* work items: tiles, times the k-slices of a split-K product */                          \
      const long tm = (M + 255) / 256 * (epi == EPI_PARTIAL && split_k > 1 ? split_k : 1);      \
      if (w192 && slot_use(tm * (N / 192)) > slot_use(tm * ((N + 255) / 256)) + 0.02)          \
        return by_epi<192, 4, 2, AT ? 3 : 2, BT ? 3 : 2>(M, N, K, A, lda, B, ldb, epi, out_t, e, split_k, s); \
      return by_epi<256, 2, 4, AT ? 3 : 2, BT ? 3 : 2>(M, N, K, A, lda, B, ldb, epi, out_t, e, split_k, s); \
    }                                                                                           \
    return by_epi<256, 2, 4, TA, TB>(M, N, K, A, lda, B, ldb, epi, out_t, e, split_k, s);      \
  }                                                                                             \
  }
