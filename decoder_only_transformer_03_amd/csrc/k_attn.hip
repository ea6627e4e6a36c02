// Causal self-attention ("GPT-2 from Scratch", CausalSelfAttention;
// "Let's reproduce GPT-2 (124M)", FlashAttention paragraph):
//   S = q k^T / sqrt(hd), S[i][j>i] = -inf, P = softmax(S), O = P v,
// computed with an online softmax over key blocks so that the T x T matrix is
// never stored; the backward pass rebuilds P from the saved row log-sum-exp.
//
// bf16, head width 64: matrix-core kernels (v_mfma_f32_32x32x16_bf16).
// fp32 (any head width <= 64): one thread per (batch, head, position).
#include "kernels.h"

#define NEG_INF (-__builtin_inff())
constexpr float LOG2E_F = 1.4426950408889634f;
constexpr float LN2_F = 0.6931471805599453f;

// ===========================================================================
// fp32 path
// ===========================================================================
template <typename T, int HD>
__global__ __launch_bounds__(128) void attn_fwd_simt(const T* __restrict__ qkv, T* __restrict__ y,
                                                     float* __restrict__ lse, int B, int Tn, int H,
                                                     int C) {
  long i = (long)blockIdx.x * 128 + threadIdx.x;
  if (i >= (long)B * H * Tn) return;
  int t = (int)(i % Tn);
  int bh = (int)(i / Tn), h = bh % H, b = bh / H;
  const long ld = 3L * C;
  const float scale = 1.0f / sqrtf((float)HD);
  const T* qr = qkv + ((long)b * Tn + t) * ld + h * HD;
  float q[HD], o[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    q[d] = ldf(qr + d) * scale;
    o[d] = 0.f;
  }
  float m = NEG_INF, l = 0.f;
  for (int j = 0; j <= t; ++j) {
    const T* kr = qkv + ((long)b * Tn + j) * ld + C + h * HD;
    float sc = 0.f;
#pragma unroll
    for (int d = 0; d < HD; ++d) sc += q[d] * ldf(kr + d);
    float mn = fmaxf(m, sc);
    float a = expf(m - mn), p = expf(sc - mn);
    l = l * a + p;
    const T* vr = kr + C;
#pragma unroll
    for (int d = 0; d < HD; ++d) o[d] = o[d] * a + p * ldf(vr + d);
    m = mn;
  }
  T* yr = y + ((long)b * Tn + t) * C + h * HD;
#pragma unroll
  for (int d = 0; d < HD; ++d) stf(yr + d, o[d] / l);
  lse[i] = m + logf(l);
}

// dQ for one (b, h, t) and D = rowsum(dO * O), which the dK/dV pass reuses.
template <typename T, int HD>
__global__ __launch_bounds__(128) void attn_bwd_dq_simt(const T* __restrict__ qkv,
                                                        const T* __restrict__ y,
                                                        const float* __restrict__ lse,
                                                        const T* __restrict__ dy,
                                                        T* __restrict__ dqkv, float* __restrict__ dbuf,
                                                        int B, int Tn, int H, int C) {
  long i = (long)blockIdx.x * 128 + threadIdx.x;
  if (i >= (long)B * H * Tn) return;
  int t = (int)(i % Tn);
  int bh = (int)(i / Tn), h = bh % H, b = bh / H;
  const long ld = 3L * C;
  const float scale = 1.0f / sqrtf((float)HD);
  const long row = (long)b * Tn + t;
  float q[HD], go[HD], dq[HD];
  float D = 0.f;
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    q[d] = ldf(qkv + row * ld + h * HD + d);
    go[d] = ldf(dy + row * C + h * HD + d);
    D += go[d] * ldf(y + row * C + h * HD + d);
    dq[d] = 0.f;
  }
  dbuf[i] = D;
  const float L = lse[i];
  for (int j = 0; j <= t; ++j) {
    const T* kr = qkv + ((long)b * Tn + j) * ld + C + h * HD;
    const T* vr = kr + C;
    float sc = 0.f, dp = 0.f;
#pragma unroll
    for (int d = 0; d < HD; ++d) {
      sc += q[d] * ldf(kr + d);
      dp += go[d] * ldf(vr + d);
    }
    float p = expf(sc * scale - L);
    float ds = p * (dp - D);
#pragma unroll
    for (int d = 0; d < HD; ++d) dq[d] += ds * ldf(kr + d);
  }
#pragma unroll
  for (int d = 0; d < HD; ++d) stf(dqkv + row * ld + h * HD + d, dq[d] * scale);
}

template <typename T, int HD>
__global__ __launch_bounds__(128) void attn_bwd_dkv_simt(const T* __restrict__ qkv,
                                                         const float* __restrict__ lse,
                                                         const T* __restrict__ dy,
                                                         const float* __restrict__ dbuf,
                                                         T* __restrict__ dqkv, int B, int Tn, int H,
                                                         int C) {
  long i = (long)blockIdx.x * 128 + threadIdx.x;
  if (i >= (long)B * H * Tn) return;
  int j = (int)(i % Tn);
  int bh = (int)(i / Tn), h = bh % H, b = bh / H;
  const long ld = 3L * C;
  const float scale = 1.0f / sqrtf((float)HD);
  const long row = (long)b * Tn + j;
  float k[HD], v[HD], dk[HD], dv[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    k[d] = ldf(qkv + row * ld + C + h * HD + d);
    v[d] = ldf(qkv + row * ld + 2 * C + h * HD + d);
    dk[d] = dv[d] = 0.f;
  }
  for (int t = j; t < Tn; ++t) {
    const long r = (long)b * Tn + t;
    const T* qr = qkv + r * ld + h * HD;
    const T* gr = dy + r * C + h * HD;
    float sc = 0.f, dp = 0.f;
#pragma unroll
    for (int d = 0; d < HD; ++d) {
      sc += ldf(qr + d) * k[d];
      dp += ldf(gr + d) * v[d];
    }
    long li = (long)bh * Tn + t;
    float p = expf(sc * scale - lse[li]);
    float ds = p * (dp - dbuf[li]);
#pragma unroll
    for (int d = 0; d < HD; ++d) {
      dv[d] += p * ldf(gr + d);
      dk[d] += ds * ldf(qr + d);
    }
  }
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    stf(dqkv + row * ld + C + h * HD + d, dk[d] * scale);
    stf(dqkv + row * ld + 2 * C + h * HD + d, dv[d]);
  }
}

// ===========================================================================
// bf16 matrix-core path, head width 64
//
// Each workgroup has 4 wavefronts; a wavefront owns 32 queries (forward, dQ)
// or 32 keys (dK/dV).  Within a 32x32 MFMA tile the lane index l maps to
// column l%32 and the half l/32 selects which 8 of the 16 contraction slots
// the lane supplies.  Scores are formed transposed where the softmax runs per
// query (S^T = K Q^T: lane <-> query, so the row max/sum are per lane plus
// one exchange with lane^32), and untransposed where the reduction runs over
// queries (S = Q K^T in the dK/dV pass: lane <-> key).  The probability tile
// stays in registers and feeds the next MFMA as its 32-wide operand: its 16
// accumulator values per lane are {8i + 4(l/32) + j}, and the other operand
// is read from a transposed LDS tile in exactly that contraction order
// (which is free to choose, since it is a sum).
// ===========================================================================
namespace {
// LDS tiles hold 64 rows x 64 bf16 (128 bytes per row) in row-major order,
// with the eight 16-byte chunks of each row permuted by xr(row).  The
// permutation keeps both read patterns free of bank conflicts: 16-byte
// fragment reads of 16 consecutive rows at one chunk, and transpose reads of
// 4 consecutive rows x 64 bytes per half-wavefront.
__device__ __forceinline__ int xr(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Rows row0 .. row0+63 of X (row stride ld, 64 columns from X) copied straight
// from global memory into the LDS tile s by the 4 wavefronts of the block,
// 16 bytes per lane.  Rows at or past nrows repeat row nrows-1 (finite data
// that the callers mask).  Completion: s_waitcnt vmcnt(0), then a barrier.
__device__ __forceinline__ void tile_load(const bf16_t* __restrict__ X, long ld, int row0,
                                          int nrows, int tid, bf16_t* s) {
  const int lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rbase = (w * 2 + j) * 8;
    const int row = rbase + (lane >> 3);
    const int c = (lane & 7) ^ xr(row);
    const int grow = row0 + row < nrows ? row0 + row : nrows - 1;
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(X + (long)grow * ld + c * 8),
        (__attribute__((address_space(3))) void*)(s + rbase * 64), 16, 0, 0);
  }
}

__device__ __forceinline__ void tile_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Work item of this workgroup: (block index along the sequence, batch*head).
// Workgroups are handed to the 8 XCDs round-robin by flat id; the ids are
// permuted so that each XCD gets a contiguous range of heads and all sequence
// blocks of a head run on one XCD, sharing its L2 for that head's K/V (or
// Q/dO).  Within a head, blocks come in the order given by `rev`.
__device__ __forceinline__ void attn_item(bool rev, int& blk, int& bh) {
  const int nb = gridDim.x, total = nb * gridDim.y;
  int id = blockIdx.y * nb + blockIdx.x;
  if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
  bh = id / nb;
  blk = rev ? nb - 1 - id % nb : id % nb;
}

// 16-byte fragment: 8 consecutive columns (chunk c) of one row.
__device__ __forceinline__ bf16x8_t frag_rows(const bf16_t* s, int row, int c) {
  return *reinterpret_cast<const bf16x8_t*>(s + row * 64 + ((c ^ xr(row)) << 3));
}

typedef short short4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 read_tr(const bf16_t* s, int row, int col) {
  const bf16_t* p = s + row * 64 + (((col >> 3) ^ xr(row)) << 3) + (col & 7);
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)((__attribute__((address_space(3))) bf16_t*)p));
  return __builtin_bit_cast(uint2, v);
}

// Operand fragment of the transposed tile: lane l supplies row d = dbase +
// l%32 of the transpose (column d of the tile) at contraction slots
// {base + 4h + 0..3, base + 8 + 4h + 0..3}, h = l/32, i.e. tile rows.  Each
// transpose read gathers, for a group of 16 lanes, a 4-row x 16-column block:
// lane t of the group addresses row t/4, columns 4(t%4)..+3, and receives
// column t of the 4 rows.
__device__ __forceinline__ bf16x8_t frag_tr(const bf16_t* s, int dbase, int base, int lane) {
  const int g = lane >> 4, t = lane & 15;
  const int row = base + 4 * (g >> 1) + (t >> 2);
  const int col = dbase + 16 * (g & 1) + 4 * (t & 3);
  const uint2 lo = read_tr(s, row, col), hi = read_tr(s, row + 8, col);
  return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Accumulator values 8u .. 8u+7 as a bf16 operand (contraction slots 16u..16u+15).
__device__ __forceinline__ bf16x8_t pack_acc(const f32x16_t& a, int u) {
  return as_bf16x8(make_uint4(pack_bf2(a[8 * u + 0], a[8 * u + 1]), pack_bf2(a[8 * u + 2], a[8 * u + 3]),
                              pack_bf2(a[8 * u + 4], a[8 * u + 5]), pack_bf2(a[8 * u + 6], a[8 * u + 7])));
}

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (results below 2^-126 flush to zero, which
// does not matter for probabilities).
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Column sums over a workgroup's 128 rows (row = 32 * wavefront + lane % 32)
// of accumulator tiles whose lane holds dims 8i + 4(lane/32) + j, through an
// LDS buffer of 128 rows x W floats; tile a of a row occupies dims 32a ..
// 32a+31, its 16-byte slots XOR-permuted by row % 8.  red_put stores one
// tile (zeros for invalid rows); after a barrier red_sum adds dim d over the
// 128 rows in a fixed order.
template <int W>
__device__ __forceinline__ void red_put(float* red, const f32x16_t& v, int a, int row, int half,
                                        bool valid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = (a * 8 + 2 * i + half) ^ (row & 7);
    *reinterpret_cast<float4*>(red + row * W + slot * 4) =
        valid ? make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3])
              : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}
template <int W>
__device__ __forceinline__ float red_sum(const float* red, int d) {
  float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int r = 0; r < 128; r += 4)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      s[u] += red[(r + u) * W + ((((d >> 2) ^ ((r + u) & 7))) << 2) + (d & 3)];
  return (s[0] + s[1]) + (s[2] + s[3]);
}

__device__ __forceinline__ float dot8(uint4 a, uint4 b) {
  float s = 0.f;
  uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s += __uint_as_float(aw[i] << 16) * __uint_as_float(bw[i] << 16);
    s += __uint_as_float(aw[i] & 0xffff0000u) * __uint_as_float(bw[i] & 0xffff0000u);
  }
  return s;
}
}  // namespace

__global__ __launch_bounds__(256) void attn_fwd_mfma(const bf16_t* __restrict__ qkv,
                                                     bf16_t* __restrict__ y,
                                                     float* __restrict__ lse, int Tn, int H, int C) {
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][64 * 64];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][64 * 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  int qb, bh;
  attn_item(true, qb, bh);  // longest rows first
  const int b = bh / H, h = bh % H;
  const long ld = 3L * C;
  const bf16_t* base = qkv + (long)b * Tn * ld;
  const bf16_t* kbase = base + C + h * 64;
  const bf16_t* vbase = base + 2 * C + h * 64;
  const int q0w = qb * 128 + w * 32;
  const int myq = q0w + l32;
  const float sl2 = 0.125f * LOG2E_F;

  bf16x8_t qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qf[kk] = as_bf16x8(myq < Tn ? *reinterpret_cast<const uint4*>(base + (long)myq * ld + h * 64 +
                                                                 kk * 16 + half * 8)
                                : make_uint4(0, 0, 0, 0));
  f32x16_t o0 = zero16(), o1 = zero16();
  float m2 = NEG_INF, ls = 0.f;
  const int kend = Tn < qb * 128 + 128 ? Tn : qb * 128 + 128;
  tile_load(kbase, ld, 0, Tn, tid, sK[0]);
  tile_load(vbase, ld, 0, Tn, tid, sV[0]);
  tile_wait();
  __syncthreads();
  int cur = 0;
  for (int k0 = 0; k0 < kend; k0 += 64, cur ^= 1) {
    const bool more = k0 + 64 < kend;
    if (more) {
      tile_load(kbase, ld, k0 + 64, Tn, tid, sK[cur ^ 1]);
      tile_load(vbase, ld, k0 + 64, Tn, tid, sV[cur ^ 1]);
    }
    if (k0 <= q0w + 31) {  // this wavefront has unmasked keys in the block
      // S^T for keys k0..k0+31 (sa) and k0+32..k0+63 (sb): two independent
      // chains; masked entries -inf
      f32x16_t sa, sb;
      auto scores = [&]() {
        sa = zero16();
        sb = zero16();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          sa = mfma(frag_rows(sK[cur], l32, kk * 2 + half), qf[kk], sa);
          sb = mfma(frag_rows(sK[cur], 32 + l32, kk * 2 + half), qf[kk], sb);
        }
        if (k0 + 63 > q0w || k0 + 63 >= Tn) {  // diagonal or ragged block
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 8 * (r >> 2) + 4 * half + (r & 3);
            sa[r] = (key > myq || key >= Tn) ? NEG_INF : sa[r];
            sb[r] = (key + 32 > myq || key + 32 >= Tn) ? NEG_INF : sb[r];
          }
        }
      };
      scores();
      // Probabilities are taken against the running reference m2 (log2
      // units) without looking for the block maximum.  Only when a block's
      // sum exceeds 2^16 -- some score rose far above m2 -- or on the first
      // block is the block rescored, its maximum taken, and O and the sum
      // rescaled to the new reference.  Probabilities stay below 2^16 or so:
      // harmless in fp32 and bf16, and the normalisation at the end is exact.
      // (key 0 is visible to every query, so after the wavefront's first
      // block, k0 == 0, every lane has a finite reference)
      const bool first = k0 == 0;
      float bs = 0.f;
      bool redo = first;
      if (!first) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sa[r] = ex2(fmaf(sa[r], sl2, -m2));
          sb[r] = ex2(fmaf(sb[r], sl2, -m2));
          bs += sa[r] + sb[r];
        }
        redo = !(bs <= 65536.0f);
      }
      if (__any(redo)) {
        if (!first) scores();
        float mx = NEG_INF;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(sa[r], sb[r]));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = fmaxf(m2, mx * sl2);
        const float alpha = first ? 0.f : ex2(m2 - mn);
        m2 = mn;
        ls *= alpha;
        o0 *= alpha;
        o1 *= alpha;
        const float ms = m2 == NEG_INF ? 0.f : m2;
        bs = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sa[r] = ex2(fmaf(sa[r], sl2, -ms));
          sb[r] = ex2(fmaf(sb[r], sl2, -ms));
          bs += sa[r] + sb[r];
        }
      }
      ls += bs;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8_t pa = pack_acc(sa, u), pb = pack_acc(sb, u);
        o0 = mfma(frag_tr(sV[cur], 0, 16 * u, lane), pa, o0);
        o1 = mfma(frag_tr(sV[cur], 32, 16 * u, lane), pa, o1);
        o0 = mfma(frag_tr(sV[cur], 0, 32 + 16 * u, lane), pb, o0);
        o1 = mfma(frag_tr(sV[cur], 32, 32 + 16 * u, lane), pb, o1);
      }
    }
    tile_wait();
    __syncthreads();
  }
  const float lt = ls + __shfl_xor(ls, 32, 64);
  const float inv = 1.0f / lt;
  if (myq < Tn) {
    bf16_t* yr = y + ((long)b * Tn + myq) * C + h * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v0[4] = {o0[4 * i] * inv, o0[4 * i + 1] * inv, o0[4 * i + 2] * inv, o0[4 * i + 3] * inv};
      float v1[4] = {o1[4 * i] * inv, o1[4 * i + 1] * inv, o1[4 * i + 2] * inv, o1[4 * i + 3] * inv};
      st4(yr + 8 * i + 4 * half, v0);
      st4(yr + 32 + 8 * i + 4 * half, v1);
    }
    if (half == 0) lse[(long)bh * Tn + myq] = (m2 + log2f(lt)) * LN2_F;
  }
}

// dQ = (P o (dP - D)) K / sqrt(hd) per block of 128 queries; also D = rowsum(dO o O).
__global__ __launch_bounds__(256) void attn_bwd_dq_mfma(const bf16_t* __restrict__ qkv,
                                                        const bf16_t* __restrict__ y,
                                                        const float* __restrict__ lse,
                                                        const bf16_t* __restrict__ dy,
                                                        bf16_t* __restrict__ dqkv,
                                                        float* __restrict__ dbuf,
                                                        float* __restrict__ bias_part, int Tn,
                                                        int H, int C) {
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][64 * 64];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][64 * 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  int qb, bh;
  attn_item(true, qb, bh);
  const int b = bh / H, h = bh % H;
  const long ld = 3L * C;
  const bf16_t* base = qkv + (long)b * Tn * ld;
  const bf16_t* dyb = dy + (long)b * Tn * C;
  const bf16_t* yb = y + (long)b * Tn * C;
  const int q0w = qb * 128 + w * 32;
  const int myq = q0w + l32;
  const float sl2 = 0.125f * LOG2E_F;

  bf16x8_t qf[4], gf[4];
  float dd = 0.f;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    uint4 q = make_uint4(0, 0, 0, 0), g = q, o = q;
    if (myq < Tn) {
      q = *reinterpret_cast<const uint4*>(base + (long)myq * ld + h * 64 + kk * 16 + half * 8);
      g = *reinterpret_cast<const uint4*>(dyb + (long)myq * C + h * 64 + kk * 16 + half * 8);
      o = *reinterpret_cast<const uint4*>(yb + (long)myq * C + h * 64 + kk * 16 + half * 8);
    }
    qf[kk] = as_bf16x8(q);
    gf[kk] = as_bf16x8(g);
    dd += dot8(g, o);
  }
  dd += __shfl_xor(dd, 32, 64);
  if (myq < Tn && half == 0) dbuf[(long)bh * Tn + myq] = dd;
  const float lse2 = myq < Tn ? lse[(long)bh * Tn + myq] * LOG2E_F : 0.f;

  f32x16_t dq0 = zero16(), dq1 = zero16();
  const int kend = Tn < qb * 128 + 128 ? Tn : qb * 128 + 128;
  const bf16_t* kbase = base + C + h * 64;
  const bf16_t* vbase = base + 2 * C + h * 64;
  tile_load(kbase, ld, 0, Tn, tid, sK[0]);
  tile_load(vbase, ld, 0, Tn, tid, sV[0]);
  tile_wait();
  __syncthreads();
  int cur = 0;
  for (int k0 = 0; k0 < kend; k0 += 64, cur ^= 1) {
    const bool more = k0 + 64 < kend;
    if (more) {
      tile_load(kbase, ld, k0 + 64, Tn, tid, sK[cur ^ 1]);
      tile_load(vbase, ld, k0 + 64, Tn, tid, sV[cur ^ 1]);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kb = k0 + 32 * s;
      if (kb > q0w + 31 || kb >= Tn) break;
      f32x16_t st = zero16(), dp = zero16();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        st = mfma(frag_rows(sK[cur], 32 * s + l32, kk * 2 + half), qf[kk], st);
        dp = mfma(frag_rows(sV[cur], 32 * s + l32, kk * 2 + half), gf[kk], dp);
      }
      if (kb + 31 > q0w || kb + 31 >= Tn) {  // diagonal or ragged block: mask
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 8 * (r >> 2) + 4 * half + (r & 3);
          const float p = (key <= myq && key < Tn) ? ex2(fmaf(st[r], sl2, -lse2)) : 0.f;
          st[r] = p * (dp[r] - dd);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) st[r] = ex2(fmaf(st[r], sl2, -lse2)) * (dp[r] - dd);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8_t pb = pack_acc(st, u);
        dq0 = mfma(frag_tr(sK[cur], 0, 32 * s + 16 * u, lane), pb, dq0);
        dq1 = mfma(frag_tr(sK[cur], 32, 32 * s + 16 * u, lane), pb, dq1);
      }
    }
    tile_wait();
    __syncthreads();
  }
  if (myq < Tn) {
    bf16_t* o = dqkv + ((long)b * Tn + myq) * ld + h * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v0[4] = {dq0[4 * i] * 0.125f, dq0[4 * i + 1] * 0.125f, dq0[4 * i + 2] * 0.125f,
                     dq0[4 * i + 3] * 0.125f};
      float v1[4] = {dq1[4 * i] * 0.125f, dq1[4 * i + 1] * 0.125f, dq1[4 * i + 2] * 0.125f,
                     dq1[4 * i + 3] * 0.125f};
      st4(o + 8 * i + 4 * half, v0);
      st4(o + 32 + 8 * i + 4 * half, v1);
    }
  }
  if (bias_part) {
    // the q part of the c_attn bias gradient: column sums of dQ over this
    // workgroup's queries, one row of partials per (sequence, query block)
    float* r0 = reinterpret_cast<float*>(sK);  // 128 x 32 floats each; K/V reads are done
    float* r1 = reinterpret_cast<float*>(sV);
    const int row = w * 32 + l32;
    red_put<32>(r0, dq0, 0, row, half, myq < Tn);
    red_put<32>(r1, dq1, 0, row, half, myq < Tn);
    __syncthreads();
    if (tid < 64)
      bias_part[((long)b * gridDim.x + qb) * 3 * C + h * 64 + tid] =
          red_sum<32>(tid < 32 ? r0 : r1, tid & 31) * 0.125f;
  }
}

// dV = P^T dO and dK = (P o (dP - D))^T Q / sqrt(hd) per block of 128 keys.
__global__ __launch_bounds__(256) void attn_bwd_dkv_mfma(const bf16_t* __restrict__ qkv,
                                                         const float* __restrict__ lse,
                                                         const bf16_t* __restrict__ dy,
                                                         const float* __restrict__ dbuf,
                                                         bf16_t* __restrict__ dqkv,
                                                         float* __restrict__ bias_part, int Tn,
                                                         int H, int C) {
  constexpr int QT = 128;  // queries staged per step (two 64-row tiles)
  __shared__ __attribute__((aligned(16))) bf16_t sQ[2][QT * 64];
  __shared__ __attribute__((aligned(16))) bf16_t sG[2][QT * 64];
  __shared__ __attribute__((aligned(16))) float sL[2][QT];
  __shared__ __attribute__((aligned(16))) float sD[2][QT];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  int kbk, bh;
  attn_item(false, kbk, bh);  // key block 0 has the most queries: dispatched first
  const int b = bh / H, h = bh % H;
  const long ld = 3L * C;
  const bf16_t* base = qkv + (long)b * Tn * ld;
  const bf16_t* dyb = dy + (long)b * Tn * C;
  const int kw0 = kbk * 128 + w * 32;
  const int mykey = kw0 + l32;
  const float sl2 = 0.125f * LOG2E_F;

  bf16x8_t kf[4], vf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    uint4 k = make_uint4(0, 0, 0, 0), v = k;
    if (mykey < Tn) {
      k = *reinterpret_cast<const uint4*>(base + (long)mykey * ld + C + h * 64 + kk * 16 + half * 8);
      v = *reinterpret_cast<const uint4*>(base + (long)mykey * ld + 2 * C + h * 64 + kk * 16 +
                                          half * 8);
    }
    kf[kk] = as_bf16x8(k);
    vf[kk] = as_bf16x8(v);
  }
  f32x16_t dv0 = zero16(), dv1 = zero16(), dk0 = zero16(), dk1 = zero16();
  const bf16_t* qbase = base + h * 64;
  const bf16_t* gbase = dyb + h * 64;
  const float* lrow = lse + (long)bh * Tn;
  const float* drow = dbuf + (long)bh * Tn;
  float ll = 0.f, dl = 0.f;
  auto load_all = [&](int q0, int buf) {
#pragma unroll
    for (int t = 0; t < QT / 64; ++t) {
      tile_load(qbase, ld, q0 + 64 * t, Tn, tid, sQ[buf] + t * 4096);
      tile_load(gbase, C, q0 + 64 * t, Tn, tid, sG[buf] + t * 4096);
    }
    if (tid < QT) {
      int q = q0 + tid;
      ll = q < Tn ? lrow[q] * LOG2E_F : 0.f;
      dl = q < Tn ? drow[q] : 0.f;
    }
  };
  auto store_all = [&](int buf) {
    tile_wait();
    if (tid < QT) {
      sL[buf][tid] = ll;
      sD[buf][tid] = dl;
    }
  };
  const int qstart = kbk * 128;
  if (qstart < Tn) {
    load_all(qstart, 0);
    store_all(0);
  }
  __syncthreads();
  int cur = 0;
  for (int q0 = qstart; q0 < Tn; q0 += QT, cur ^= 1) {
    const bool more = q0 + QT < Tn;
    if (more) load_all(q0 + QT, cur ^ 1);
#pragma unroll
    for (int s = 0; s < QT / 32; ++s) {
      const int qs = q0 + 32 * s;
      if (qs + 31 < kw0 || qs >= Tn) continue;
      f32x16_t st = zero16(), dp = zero16();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        st = mfma(frag_rows(sQ[cur], 32 * s + l32, kk * 2 + half), kf[kk], st);
        dp = mfma(frag_rows(sG[cur], 32 * s + l32, kk * 2 + half), vf[kk], dp);
      }
      // log-sum-exp and D of this lane's 16 queries: four runs of 4
      float lq[16], dd[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qi = 32 * s + 8 * g + 4 * half;
        const float4 a = *reinterpret_cast<const float4*>(&sL[cur][qi]);
        const float4 c = *reinterpret_cast<const float4*>(&sD[cur][qi]);
        lq[4 * g] = a.x; lq[4 * g + 1] = a.y; lq[4 * g + 2] = a.z; lq[4 * g + 3] = a.w;
        dd[4 * g] = c.x; dd[4 * g + 1] = c.y; dd[4 * g + 2] = c.z; dd[4 * g + 3] = c.w;
      }
      f32x16_t pv;
      if (qs < kw0 + 31 || qs + 31 >= Tn) {  // some (query, key) pair masked
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = q0 + 32 * s + 8 * (r >> 2) + 4 * half + (r & 3);
          const float p = (mykey <= q && q < Tn) ? ex2(fmaf(st[r], sl2, -lq[r])) : 0.f;
          pv[r] = p;
          st[r] = p * (dp[r] - dd[r]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = ex2(fmaf(st[r], sl2, -lq[r]));
          pv[r] = p;
          st[r] = p * (dp[r] - dd[r]);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8_t pp = pack_acc(pv, u), ps = pack_acc(st, u);
        dv0 = mfma(frag_tr(sG[cur], 0, 32 * s + 16 * u, lane), pp, dv0);
        dv1 = mfma(frag_tr(sG[cur], 32, 32 * s + 16 * u, lane), pp, dv1);
        dk0 = mfma(frag_tr(sQ[cur], 0, 32 * s + 16 * u, lane), ps, dk0);
        dk1 = mfma(frag_tr(sQ[cur], 32, 32 * s + 16 * u, lane), ps, dk1);
      }
    }
    if (more) store_all(cur ^ 1);
    __syncthreads();
  }
  if (mykey < Tn) {
    bf16_t* o = dqkv + ((long)b * Tn + mykey) * ld + h * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float k0[4] = {dk0[4 * i] * 0.125f, dk0[4 * i + 1] * 0.125f, dk0[4 * i + 2] * 0.125f,
                     dk0[4 * i + 3] * 0.125f};
      float k1[4] = {dk1[4 * i] * 0.125f, dk1[4 * i + 1] * 0.125f, dk1[4 * i + 2] * 0.125f,
                     dk1[4 * i + 3] * 0.125f};
      float v0[4] = {dv0[4 * i], dv0[4 * i + 1], dv0[4 * i + 2], dv0[4 * i + 3]};
      float v1[4] = {dv1[4 * i], dv1[4 * i + 1], dv1[4 * i + 2], dv1[4 * i + 3]};
      st4(o + C + 8 * i + 4 * half, k0);
      st4(o + C + 32 + 8 * i + 4 * half, k1);
      st4(o + 2 * C + 8 * i + 4 * half, v0);
      st4(o + 2 * C + 32 + 8 * i + 4 * half, v1);
    }
  }
  if (bias_part) {
    // the k and v parts of the c_attn bias gradient: column sums of dK and dV
    // over this workgroup's keys, one row of partials per (sequence, key block)
    float* rk = reinterpret_cast<float*>(sQ);  // 128 x 64 floats each; Q/dO reads are done
    float* rv = reinterpret_cast<float*>(sG);
    const int row = w * 32 + l32;
    const bool ok = mykey < Tn;
    red_put<64>(rk, dk0, 0, row, half, ok);
    red_put<64>(rk, dk1, 1, row, half, ok);
    red_put<64>(rv, dv0, 0, row, half, ok);
    red_put<64>(rv, dv1, 1, row, half, ok);
    __syncthreads();
    if (tid < 128) {
      float* out = bias_part + ((long)b * gridDim.x + kbk) * 3 * C + h * 64;
      if (tid < 64) out[C + tid] = red_sum<64>(rk, tid) * 0.125f;
      else out[2 * C + tid - 64] = red_sum<64>(rv, tid - 64);
    }
  }
}

// ===========================================================================
// Decoding with a key/value cache: one new position per sequence.
// ===========================================================================

// The key and value parts of rows t of qkv ((B*T, 3C), sequence b at rows
// b*T .. b*T+T-1) into the cache (B, bs, 2C) at positions pos0 + t.
template <typename T>
__global__ __launch_bounds__(256) void kv_append_kernel(const T* __restrict__ qkv,
                                                        T* __restrict__ cache, int Tn, int pos0,
                                                        int bs, int C, long rows) {
  const long row = (long)blockIdx.x;
  if (row >= rows) return;
  const long b = row / Tn, t = row % Tn;
  const T* src = qkv + row * 3L * C + C;
  T* dst = cache + (b * bs + pos0 + t) * 2L * C;
  for (int c = threadIdx.x; c < 2 * C; c += 256) dst[c] = src[c];
}

// Attention of the query of each (b, h) -- the single new position p -- over
// the cached keys and values of positions 0 .. p (all visible: they precede
// or are the query).  One workgroup per (b, h); fp32 arithmetic.  q is row b
// of qkv (B, 3C); y row b of (B, C).
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_decode_kernel(const T* __restrict__ qkv,
                                                          const T* __restrict__ cache,
                                                          T* __restrict__ y, int p, int bs, int H,
                                                          int C) {
  extern __shared__ float dsh[];  // p+1 scores, then 256 reduction slots
  float* sc = dsh;
  float* red = dsh + ((p + 1 + 63) & ~63);
  __shared__ float qs[HD];
  const int bh = blockIdx.x, b = bh / H, h = bh % H, tid = threadIdx.x;
  const float scale = 1.0f / sqrtf((float)HD);
  if (tid < HD) qs[tid] = ldf(qkv + (long)b * 3 * C + h * HD + tid) * scale;
  __syncthreads();
  const T* kb = cache + (long)b * bs * 2 * C + h * HD;
  const T* vb = kb + C;
  float mx = -__builtin_inff();
  for (int j = tid; j <= p; j += 256) {
    const T* kr = kb + (long)j * 2 * C;
    float s = 0.f;
#pragma unroll 8
    for (int d = 0; d < HD; ++d) s += qs[d] * ldf(kr + d);
    sc[j] = s;
    mx = fmaxf(mx, s);
  }
  red[tid] = mx;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
    __syncthreads();
  }
  mx = red[0];
  __syncthreads();
  float sum = 0.f;
  for (int j = tid; j <= p; j += 256) {
    const float e = __expf(sc[j] - mx);
    sc[j] = e;
    sum += e;
  }
  red[tid] = sum;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  const float inv = 1.0f / red[0];
  __syncthreads();
  // O[d] = sum_j P_j V_j[d]: lanes of one group cover the HD dimensions,
  // groups take every G-th position; the groups' sums meet in LDS
  constexpr int G = 256 / HD;
  const int d = tid % HD, g = tid / HD;
  float acc = 0.f;
  for (int j = g; j <= p; j += G) acc += sc[j] * ldf(vb + (long)j * 2 * C + d);
  red[tid] = acc;
  __syncthreads();
  if (tid < HD) {
    float o = 0.f;
    for (int k = 0; k < G; ++k) o += red[k * HD + tid];
    stf(y + (long)b * C + h * HD + tid, o * inv);
  }
}

// bf16, head width 64: the same attention with the new position's key and
// value also appended to the cache (each (b, h) workgroup writes its head's
// 64 + 64 values), in one launch.  Eight lanes share a position, each with 8
// of the 64 dimensions (16-byte loads of whole 128-byte key and value rows);
// the 256 threads hold 32 positions at a time and issue the key and value
// loads of up to DEC_NB positions per thread before using any.  Each group of
// eight keeps an online softmax (running maximum, sum, and its 8 dimensions
// of the weighted values, on exp2 with log2(e)/sqrt(64) folded into q); the
// 32 groups are merged in a fixed order through LDS.  Position p's own key
// and value come from the qkv row, not from the cache being written.
constexpr int DEC_NB = 4;
__global__ __launch_bounds__(256) void attn_decode_bf16_kernel(const bf16_t* __restrict__ qkv,
                                                               bf16_t* __restrict__ cache,
                                                               bf16_t* __restrict__ y, int p,
                                                               int bs, int H, int C) {
  constexpr int HD = 64;
  __shared__ float gm[32], gl[32];
  __shared__ float go[32][HD + 1];
  const int bh = blockIdx.x, b = bh / H, h = bh % H, tid = threadIdx.x;
  const int ps = tid >> 3, dc = tid & 7;  // position slot, 8-dimension chunk
  const bf16_t* qrow = qkv + (long)b * 3 * C + h * HD;
  const uint4 kp = *reinterpret_cast<const uint4*>(qrow + C + 8 * dc);
  const uint4 vp = *reinterpret_cast<const uint4*>(qrow + 2 * C + 8 * dc);
  bf16_t* kc = cache + (long)b * bs * 2 * C + h * HD + 8 * dc;  // key row 0, this chunk
  if (ps == 0) {
    *reinterpret_cast<uint4*>(kc + (long)p * 2 * C) = kp;
    *reinterpret_cast<uint4*>(kc + (long)p * 2 * C + C) = vp;
  }
  float q[8];
  {
    const uint4 qv = *reinterpret_cast<const uint4*>(qrow + 8 * dc);
    const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
    const float sc = 0.125f * 1.4426950408889634f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[2 * i] = __uint_as_float(w[i] << 16) * sc;
      q[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u) * sc;
    }
  }
  float m = -__builtin_inff(), l = 0.f, o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
  for (int j0 = 0; j0 <= p; j0 += 32 * DEC_NB) {
    uint4 kv[DEC_NB], vv[DEC_NB];
#pragma unroll
    for (int i = 0; i < DEC_NB; ++i) {
      const int j = j0 + ps + 32 * i;
      if (j < p) {
        kv[i] = *reinterpret_cast<const uint4*>(kc + (long)j * 2 * C);
        vv[i] = *reinterpret_cast<const uint4*>(kc + (long)j * 2 * C + C);
      } else {
        kv[i] = kp;
        vv[i] = vp;
      }
    }
#pragma unroll
    for (int i = 0; i < DEC_NB; ++i) {
      const int j = j0 + ps + 32 * i;
      const uint32_t kw[4] = {kv[i].x, kv[i].y, kv[i].z, kv[i].w};
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        s = fmaf(q[2 * t], __uint_as_float(kw[t] << 16), s);
        s = fmaf(q[2 * t + 1], __uint_as_float(kw[t] & 0xffff0000u), s);
      }
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      s += __shfl_xor(s, 4, 64);
      if (j <= p) {  // the same for the 8 lanes of the group
        const float mn = fmaxf(m, s);
        const float a = __builtin_amdgcn_exp2f(m - mn), e = __builtin_amdgcn_exp2f(s - mn);
        l = l * a + e;
        const uint32_t vw[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          o[2 * t] = o[2 * t] * a + e * __uint_as_float(vw[t] << 16);
          o[2 * t + 1] = o[2 * t + 1] * a + e * __uint_as_float(vw[t] & 0xffff0000u);
        }
        m = mn;
      }
    }
  }
  // merge the 32 groups: slots past p (possible when p < 31) hold m = -inf
  if (dc == 0) {
    gm[ps] = m;
    gl[ps] = l;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) go[ps][8 * dc + i] = o[i];
  __syncthreads();
  if (tid < HD) {
    float M = gm[0];
    for (int g = 1; g < 32; ++g) M = fmaxf(M, gm[g]);
    float L = 0.f, O = 0.f;
    for (int g = 0; g < 32; ++g) {
      if (gm[g] == -__builtin_inff()) continue;
      const float f = __builtin_amdgcn_exp2f(gm[g] - M);
      L += gl[g] * f;
      O += go[g][tid] * f;
    }
    stf(y + (long)b * C + h * HD + tid, O / L);
  }
}

// ===========================================================================
// launchers
// ===========================================================================
template <typename T>
static hipError_t simt_fwd(const void* qkv, void* y, float* lse, int B, int Tn, int H, int hd,
                           hipStream_t s) {
  long n = (long)B * H * Tn;
  unsigned g = (unsigned)((n + 127) / 128);
  int C = H * hd;
  if (hd == 32)
    attn_fwd_simt<T, 32><<<g, 128, 0, s>>>((const T*)qkv, (T*)y, lse, B, Tn, H, C);
  else
    attn_fwd_simt<T, 64><<<g, 128, 0, s>>>((const T*)qkv, (T*)y, lse, B, Tn, H, C);
  return hipGetLastError();
}

template <typename T>
static hipError_t simt_bwd(const void* qkv, const void* y, const float* lse, const void* dy,
                           void* dqkv, float* dbuf, int B, int Tn, int H, int hd, hipStream_t s) {
  long n = (long)B * H * Tn;
  unsigned g = (unsigned)((n + 127) / 128);
  int C = H * hd;
  if (hd == 32) {
    attn_bwd_dq_simt<T, 32><<<g, 128, 0, s>>>((const T*)qkv, (const T*)y, lse, (const T*)dy,
                                              (T*)dqkv, dbuf, B, Tn, H, C);
    attn_bwd_dkv_simt<T, 32><<<g, 128, 0, s>>>((const T*)qkv, lse, (const T*)dy, dbuf, (T*)dqkv,
                                               B, Tn, H, C);
  } else {
    attn_bwd_dq_simt<T, 64><<<g, 128, 0, s>>>((const T*)qkv, (const T*)y, lse, (const T*)dy,
                                              (T*)dqkv, dbuf, B, Tn, H, C);
    attn_bwd_dkv_simt<T, 64><<<g, 128, 0, s>>>((const T*)qkv, lse, (const T*)dy, dbuf, (T*)dqkv,
                                               B, Tn, H, C);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd(DType t, const void* qkv, void* y, float* lse, int B, int Tn, int H,
                           int hd, hipStream_t s) {
  if (t == DT_BF16) {
    if (hd != 64) return hipErrorInvalidValue;
    dim3 grid((Tn + 127) / 128, B * H);
    attn_fwd_mfma<<<grid, 256, 0, s>>>((const bf16_t*)qkv, (bf16_t*)y, lse, Tn, H, H * 64);
    return hipGetLastError();
  }
  if (hd != 32 && hd != 64) return hipErrorInvalidValue;
  return simt_fwd<float>(qkv, y, lse, B, Tn, H, hd, s);
}

hipError_t launch_attn_bwd(DType t, const void* qkv, const void* y, const float* lse,
                           const void* dy, void* dqkv, float* dbuf, int B, int Tn, int H, int hd,
                           float* bias_part, hipStream_t s) {
  if (t == DT_BF16) {
    if (hd != 64) return hipErrorInvalidValue;
    dim3 grid((Tn + 127) / 128, B * H);
    int C = H * 64;
    attn_bwd_dq_mfma<<<grid, 256, 0, s>>>((const bf16_t*)qkv, (const bf16_t*)y, lse,
                                          (const bf16_t*)dy, (bf16_t*)dqkv, dbuf, bias_part, Tn,
                                          H, C);
    attn_bwd_dkv_mfma<<<grid, 256, 0, s>>>((const bf16_t*)qkv, lse, (const bf16_t*)dy, dbuf,
                                           (bf16_t*)dqkv, bias_part, Tn, H, C);
    return hipGetLastError();
  }
  if ((hd != 32 && hd != 64) || bias_part) return hipErrorInvalidValue;
  return simt_bwd<float>(qkv, y, lse, dy, dqkv, dbuf, B, Tn, H, hd, s);
}

hipError_t launch_kv_append(DType t, const void* qkv, void* cache, int B, int Tn, int pos0, int bs,
                            int C, hipStream_t s) {
  const long rows = (long)B * Tn;
  if (rows <= 0) return hipSuccess;
  if (t == DT_BF16)
    kv_append_kernel<bf16_t><<<(unsigned)rows, 256, 0, s>>>((const bf16_t*)qkv, (bf16_t*)cache,
                                                            Tn, pos0, bs, C, rows);
  else
    kv_append_kernel<float><<<(unsigned)rows, 256, 0, s>>>((const float*)qkv, (float*)cache, Tn,
                                                           pos0, bs, C, rows);
  return hipGetLastError();
}

hipError_t launch_attn_decode(DType t, const void* qkv, void* cache, void* y, int B, int p, int bs,
                              int H, int hd, hipStream_t s) {
  if (p < 0 || p >= bs || p >= ATTN_DECODE_MAX_POS) return hipErrorInvalidValue;
  const int C = H * hd;
  const unsigned g = (unsigned)(B * H);
  if (t == DT_BF16) {
    if (hd != 64) return hipErrorInvalidValue;
    attn_decode_bf16_kernel<<<g, 256, 0, s>>>((const bf16_t*)qkv, (bf16_t*)cache, (bf16_t*)y, p,
                                              bs, H, C);
    return hipGetLastError();
  }
  if (hd != 64 && hd != 32) return hipErrorInvalidValue;
  hipError_t r = launch_kv_append(t, qkv, cache, B, 1, p, bs, C, s);
  if (r != hipSuccess) return r;
  const size_t lds = (size_t)(((p + 1 + 63) & ~63) + 256) * sizeof(float);
  if (hd == 64)
    attn_decode_kernel<float, 64><<<g, 256, lds, s>>>((const float*)qkv, (const float*)cache,
                                                      (float*)y, p, bs, H, C);
  else
    attn_decode_kernel<float, 32><<<g, 256, lds, s>>>((const float*)qkv, (const float*)cache,
                                                      (float*)y, p, bs, H, C);
  return hipGetLastError();
}
