// Bandwidth-bound kernels of the GPT-2 step: embedding gather / scatter-add,
// LayerNorm forward / backward, fused softmax cross-entropy, bias-gradient
// column sums, global gradient norm and AdamW.  All are row- or
// element-parallel with wavefront (64-lane) reductions and 16-byte accesses.
#include "kernels.h"

// ---------------------------------------------------------------------------
// x[b,t,:] = wte[idx[b,t],:] + wpe[t,:]        ("GPT-2 from Scratch", Embeddings)
// One wavefront per row.  Out-of-range ids set a flag and read row 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void embed_fwd_kernel(const int32_t* __restrict__ idx_in,
                                                        int32_t* __restrict__ idx_saved,
                                                        const float* __restrict__ wte,
                                                        const float* __restrict__ wpe,
                                                        float* __restrict__ x, int T, int C, int Vp,
                                                        long rows, int* err) {
  long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (row >= rows) return;
  int t = (int)(row % T);
  int id = idx_in[row];
  if (id < 0 || id >= Vp) {
    if (lane == 0) atomicOr(err, ERRF_IDX);
    id = 0;
  }
  if (lane == 0) idx_saved[row] = id;
  const float* a = wte + (long)id * C;
  const float* p = wpe + (long)t * C;
  float* o = x + row * C;
  for (int c = lane * 4; c < C; c += 256) {
    float4 u = *reinterpret_cast<const float4*>(a + c);
    float4 w = *reinterpret_cast<const float4*>(p + c);
    *reinterpret_cast<float4*>(o + c) = make_float4(u.x + w.x, u.y + w.y, u.z + w.z, u.w + w.w);
  }
}

// dwte[idx[p],:] += dx[p,:]  (adds onto the lm_head part already there: the
// tied weight's gradient is the sum of both uses, "Weight tying").
__global__ __launch_bounds__(256) void embed_bwd_wte_kernel(const int32_t* __restrict__ idx,
                                                            const float* __restrict__ dx,
                                                            float* __restrict__ dwte, int C,
                                                            long rows) {
  long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (row >= rows) return;
  int id = idx[row];
  const float* s = dx + row * C;
  float* d = dwte + (long)id * C;
  for (int c = lane * 4; c < C; c += 256) {
    float4 v = *reinterpret_cast<const float4*>(s + c);
    atomicAdd(d + c + 0, v.x);
    atomicAdd(d + c + 1, v.y);
    atomicAdd(d + c + 2, v.z);
    atomicAdd(d + c + 3, v.w);
  }
}

// dwpe[t,c] += sum_b dx[b,t,c]   (deterministic: one thread per (t, c))
__global__ __launch_bounds__(256) void embed_bwd_wpe_kernel(const float* __restrict__ dx,
                                                            float* __restrict__ dwpe, int B, int T,
                                                            int C) {
  long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)T * C) return;
  float s = 0.f;
  for (int b = 0; b < B; ++b) s += dx[(long)b * T * C + i];
  dwpe[i] += s;
}

// ---------------------------------------------------------------------------
// LayerNorm forward: y = (x - mean) * rstd * w + b, rstd = 1/sqrt(var + 1e-5),
// biased variance over C.  One wavefront per row, the row kept in registers.
// ---------------------------------------------------------------------------
constexpr int LN_MAXV = 8;  // float4 per lane: C <= 2048

template <typename TO>
__global__ __launch_bounds__(256) void layernorm_fwd_kernel(const float* __restrict__ x,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ b,
                                                            TO* __restrict__ y,
                                                            float* __restrict__ mean_out,
                                                            float* __restrict__ rstd_out,
                                                            long rows, int C) {
  long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* xr = x + row * C;
  float v[LN_MAXV][4];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    int c = (i * 64 + lane) * 4;
    if (c < C) {
      ld4(xr + c, v[i]);
      s += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
    }
  }
  float mean = wave_sum(s) / (float)C;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    int c = (i * 64 + lane) * 4;
    if (c < C) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float d = v[i][j] - mean;
        q += d * d;
      }
    }
  }
  float var = wave_sum(q) / (float)C;
  float rstd = 1.0f / sqrtf(var + 1e-5f);
  TO* yr = y + row * C;
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    int c = (i * 64 + lane) * 4;
    if (c < C) {
      float g[4], bb[4], o[4];
      ld4(w + c, g);
      ld4(b + c, bb);
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = (v[i][j] - mean) * rstd * g[j] + bb[j];
      st4(yr + c, o);
    }
  }
  if (lane == 0) {
    mean_out[row] = mean;
    rstd_out[row] = rstd;
  }
}

// ---------------------------------------------------------------------------
// LayerNorm backward.  With xhat = (x - mean) rstd and d = dy * w:
//   dx = rstd (d - mean(d) - xhat mean(d xhat)),  dw = sum dy xhat, db = sum dy.
// dres = dx (accumulate = 0) or dres += dx; an optional bf16 copy of the new
// dres feeds the next bf16 GEMM.  dw/db: per-block partial sums, reduced by
// colsum_partials_kernel (deterministic).
// ---------------------------------------------------------------------------
template <typename TB>
__global__ __launch_bounds__(256) void layernorm_bwd_kernel(
    const float* __restrict__ dy, const float* __restrict__ x, const float* __restrict__ mean,
    const float* __restrict__ rstd, const float* __restrict__ w, float* __restrict__ dres,
    TB* __restrict__ dres_copy, int accumulate, float* __restrict__ partial, long rows, int C,
    int rows_per_block) {
  extern __shared__ float sred[];  // [4][2C]
  int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float dg[LN_MAXV][4], db[LN_MAXV][4], wv[LN_MAXV][4];
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    int c = (i * 64 + lane) * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) dg[i][j] = db[i][j] = 0.f;
    if (c < C) ld4(w + c, wv[i]);
  }
  long r0 = (long)blockIdx.x * rows_per_block;
  long r1 = r0 + rows_per_block < rows ? r0 + rows_per_block : rows;
  for (long row = r0 + wave; row < r1; row += 4) {
    float mu = mean[row], rs = rstd[row];
    float g[LN_MAXV][4], xh[LN_MAXV][4];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
      int c = (i * 64 + lane) * 4;
      if (c < C) {
        float xv[4];
        ld4(dy + row * C + c, g[i]);
        ld4(x + row * C + c, xv);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xh[i][j] = (xv[j] - mu) * rs;
          dg[i][j] += g[i][j] * xh[i][j];
          db[i][j] += g[i][j];
          float d = g[i][j] * wv[i][j];
          g[i][j] = d;
          s1 += d;
          s2 += d * xh[i][j];
        }
      }
    }
    s1 = wave_sum(s1) / (float)C;
    s2 = wave_sum(s2) / (float)C;
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
      int c = (i * 64 + lane) * 4;
      if (c < C) {
        float o[4];
        float* dr = dres + row * C + c;
        if (accumulate) ld4(dr, o);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float dx = rs * (g[i][j] - s1 - xh[i][j] * s2);
          o[j] = accumulate ? o[j] + dx : dx;
        }
        st4(dr, o);
        if (dres_copy) st4(dres_copy + row * C + c, o);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    int c = (i * 64 + lane) * 4;
    if (c < C) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sred[wave * 2 * C + c + j] = dg[i][j];
        sred[wave * 2 * C + C + c + j] = db[i][j];
      }
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < 2 * C; c += 256) {
    float s = sred[c] + sred[2 * C + c] + sred[4 * C + c] + sred[6 * C + c];
    partial[(long)blockIdx.x * 2 * C + c] = s;
  }
}

// out[c] += sum_p partial[p][c]   (one thread per column, fixed order)
__global__ __launch_bounds__(256) void colsum_partials_kernel(const float* __restrict__ partial,
                                                              int nparts, int width,
                                                              float* __restrict__ out0,
                                                              float* __restrict__ out1,
                                                              int split) {
  int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= width) return;
  float s = 0.f;
  for (int p = 0; p < nparts; ++p) s += partial[(long)p * width + c];
  if (c < split) out0[c] += s;
  else out1[c - split] += s;
}

// Column sums of a (rows x N) matrix into per-split partials: bias gradients.
template <typename T>
__global__ __launch_bounds__(256) void colsum_kernel(const T* __restrict__ X, long rows, int N,
                                                     long ldx, float* __restrict__ partial,
                                                     long rows_per_split) {
  int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  long r0 = (long)blockIdx.y * rows_per_split;
  long r1 = r0 + rows_per_split < rows ? r0 + rows_per_split : rows;
  float s = 0.f;
  for (long r = r0; r < r1; ++r) s += ldf(X + r * ldx + n);
  partial[(long)blockIdx.y * N + n] = s;
}

// ---------------------------------------------------------------------------
// Cross-entropy with ignore_index = -1, fused with its gradient.
// ---------------------------------------------------------------------------
// n_valid = #{targets != -1}; flags targets outside {-1} U [0, Vp).
__global__ __launch_bounds__(1024) void count_valid_kernel(const int32_t* __restrict__ tgt,
                                                           long rows, int Vp,
                                                           int* __restrict__ n_valid, int* err) {
  __shared__ int s[16];
  int cnt = 0, bad = 0;
  for (long i = threadIdx.x; i < rows; i += 1024) {
    int t = tgt[i];
    if (t != -1) {
      ++cnt;
      if (t < 0 || t >= Vp) bad = 1;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    cnt += __shfl_xor(cnt, o, 64);
    bad |= __shfl_xor(bad, o, 64);
  }
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = cnt | (bad << 30);
  __syncthreads();
  if (threadIdx.x == 0) {
    int c = 0, b = 0;
    for (int i = 0; i < 16; ++i) {
      c += s[i] & ((1 << 30) - 1);
      b |= s[i] >> 30;
    }
    *n_valid = c;
    if (b) atomicOr(err, ERRF_TARGET);
  }
}

// Eight consecutive elements of a logits row held in registers.
template <typename T> struct Row8;
template <> struct Row8<bf16_t> {
  uint4 r;
  __device__ void load(const bf16_t* p) { r = *reinterpret_cast<const uint4*>(p); }
  __device__ float get(int j) const {
    uint32_t w = j < 2 ? r.x : j < 4 ? r.y : j < 6 ? r.z : r.w;
    return (j & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
  __device__ static void store(bf16_t* p, const float v[8]) {
    *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]),
                                              pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7]));
  }
};
template <> struct Row8<float> {
  float4 a, b;
  __device__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ float get(int j) const {
    switch (j) {
      case 0: return a.x; case 1: return a.y; case 2: return a.z; case 3: return a.w;
      case 4: return b.x; case 5: return b.y; case 6: return b.z; default: return b.w;
    }
  }
  __device__ static void store(float* p, const float v[8]) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};

__device__ __forceinline__ float block_reduce_256(float v, bool is_max, float* s4) {
  v = is_max ? wave_max(v) : wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s4[threadIdx.x >> 6] = v;
  __syncthreads();
  return is_max ? fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]))
                : (s4[0] + s4[1]) + (s4[2] + s4[3]);
}

// One workgroup per row; the row is read once into registers, its
// log-sum-exp formed, and the row is overwritten with
//   d(loss)/d(logits) = (softmax - onehot(target)) / n_valid   (0 if ignored).
// Padded vocabulary columns take part like real ones.
template <typename T, int MAXCH>
__global__ __launch_bounds__(256) void xent_fused_kernel(T* __restrict__ logits,
                                                         const int32_t* __restrict__ targets,
                                                         const int* __restrict__ n_valid,
                                                         float* __restrict__ row_loss, int Vp) {
  __shared__ float s4[4];
  long row = blockIdx.x;
  T* lr = logits + row * (long)Vp;
  int tgt = targets[row];
  bool valid = tgt != -1;
  if (tgt < 0 || tgt >= Vp) tgt = -1;  // out-of-range already flagged by count_valid
  int nchunks = Vp >> 3;
  Row8<T> v[MAXCH];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < MAXCH; ++i) {
    int ch = i * 256 + threadIdx.x;
    if (ch < nchunks) {
      v[i].load(lr + ch * 8);
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = fmaxf(mx, v[i].get(j));
    }
  }
  mx = block_reduce_256(mx, true, s4);
  float sum = 0.f, xt = 0.f;
#pragma unroll
  for (int i = 0; i < MAXCH; ++i) {
    int ch = i * 256 + threadIdx.x;
    if (ch < nchunks) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float e = v[i].get(j);
        sum += __expf(e - mx);
        if (ch * 8 + j == tgt) xt = e;
      }
    }
  }
  sum = block_reduce_256(sum, false, s4);
  xt = block_reduce_256(xt, false, s4);  // exactly one thread holds a non-zero term
  float lse = mx + __logf(sum);
  int nv = *n_valid;
  float inv = nv > 0 ? 1.0f / (float)nv : 0.f;
  float scale = valid ? inv : 0.f;
#pragma unroll
  for (int i = 0; i < MAXCH; ++i) {
    int ch = i * 256 + threadIdx.x;
    if (ch < nchunks) {
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float p = __expf(v[i].get(j) - lse);
        o[j] = (p - (ch * 8 + j == tgt ? 1.0f : 0.0f)) * scale;
      }
      Row8<T>::store(lr + ch * 8, o);
    }
  }
  if (threadIdx.x == 0) row_loss[row] = valid ? lse - xt : 0.f;
}

// loss = sum(row_loss) / n_valid  (0 when no position is valid); fp64 sum.
__global__ __launch_bounds__(1024) void loss_reduce_kernel(const float* __restrict__ row_loss,
                                                           long rows,
                                                           const int* __restrict__ n_valid,
                                                           float* __restrict__ loss) {
  __shared__ double s[16];
  double a = 0.0;
  for (long i = threadIdx.x; i < rows; i += 1024) a += (double)row_loss[i];
  a = wave_sum_d(a);
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int i = 0; i < 16; ++i) t += s[i];
    int nv = *n_valid;
    *loss = nv > 0 ? (float)(t / nv) : 0.f;
  }
}

// ---------------------------------------------------------------------------
// Global gradient norm ("Gradient clipping"): sum of squares per block in
// fp64, then one block finishes the norm and the clip coefficient
// min(1, max_norm / (norm + 1e-6)).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void sumsq_kernel(const float* __restrict__ g, long n4,
                                                    double* __restrict__ partial) {
  __shared__ double s[4];
  double a = 0.0;
  const float4* g4 = reinterpret_cast<const float4*>(g);
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long)gridDim.x * 256) {
    float4 v = g4[i];
    a += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
  }
  a = wave_sum_d(a);
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = (s[0] + s[1]) + (s[2] + s[3]);
}

__global__ __launch_bounds__(256) void norm_finish_kernel(const double* __restrict__ partial,
                                                          int nparts, float max_norm,
                                                          float* __restrict__ norm_out,
                                                          float* __restrict__ clip_out) {
  __shared__ double s[4];
  double a = 0.0;
  for (int i = threadIdx.x; i < nparts; i += 256) a += partial[i];
  a = wave_sum_d(a);
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    double nrm = sqrt((s[0] + s[1]) + (s[2] + s[3]));
    double c = (double)max_norm / (nrm + 1e-6);
    *norm_out = (float)nrm;
    *clip_out = (float)(c < 1.0 ? c : 1.0);
  }
}

// ---------------------------------------------------------------------------
// AdamW over the flat parameter vector, one workgroup per chunk; a chunk
// never crosses a tensor boundary and carries that tensor's decay flag.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void adamw_kernel(const AdamChunk* __restrict__ chunks,
                                                    float* __restrict__ p,
                                                    const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    bf16_t* __restrict__ shadow,
                                                    const float* __restrict__ clip, float lr,
                                                    float b1, float b2, float eps, float wd,
                                                    float step_size, float inv_sqrt_bc2) {
  AdamChunk ck = chunks[blockIdx.x];
  float c = *clip;
  float decay = (ck.flags & 1) ? 1.0f - lr * wd : 1.0f;
  float4* p4 = reinterpret_cast<float4*>(p + ck.start);
  const float4* g4 = reinterpret_cast<const float4*>(g + ck.start);
  float4* m4 = reinterpret_cast<float4*>(m + ck.start);
  float4* v4 = reinterpret_cast<float4*>(v + ck.start);
  int n4 = ck.len >> 2;
  for (int i = threadIdx.x; i < n4; i += 256) {
    float4 pp = p4[i], gg = g4[i], mm = m4[i], vv = v4[i];
    float P[4] = {pp.x, pp.y, pp.z, pp.w}, G[4] = {gg.x, gg.y, gg.z, gg.w};
    float M[4] = {mm.x, mm.y, mm.z, mm.w}, V[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float gj = G[j] * c;
      P[j] *= decay;
      M[j] = b1 * M[j] + (1.0f - b1) * gj;
      V[j] = b2 * V[j] + (1.0f - b2) * gj * gj;
      P[j] -= step_size * M[j] / (sqrtf(V[j]) * inv_sqrt_bc2 + eps);
    }
    p4[i] = make_float4(P[0], P[1], P[2], P[3]);
    m4[i] = make_float4(M[0], M[1], M[2], M[3]);
    v4[i] = make_float4(V[0], V[1], V[2], V[3]);
    if (shadow) st4(shadow + ck.start + 4 * (long)i, P);
  }
}

// ---------------------------------------------------------------------------
// small utilities
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ p, long n, float val) {
  long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  long stride = (long)gridDim.x * 256 * 4;
  for (; i < n; i += stride) {
    if (i + 4 <= n) *reinterpret_cast<float4*>(p + i) = make_float4(val, val, val, val);
    else
      for (long j = i; j < n; ++j) p[j] = val;
  }
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ s,
                                                          bf16_t* __restrict__ d, long n) {
  long i = (long)blockIdx.x * 256 + threadIdx.x;
  for (; i < n; i += (long)gridDim.x * 256) d[i] = f2bf(s[i]);
}

__global__ __launch_bounds__(256) void bf16_to_f32_kernel(const bf16_t* __restrict__ s,
                                                          float* __restrict__ d, long n) {
  long i = (long)blockIdx.x * 256 + threadIdx.x;
  for (; i < n; i += (long)gridDim.x * 256) d[i] = bf2f(s[i]);
}

// ===========================================================================
// launchers
// ===========================================================================
static inline unsigned nblk(long n, int per) { return (unsigned)((n + per - 1) / per); }

hipError_t launch_embed_fwd(const int32_t* idx_in, int32_t* idx_saved, const float* wte,
                            const float* wpe, float* x, int B, int T, int C, int Vp, int* err,
                            hipStream_t s) {
  long rows = (long)B * T;
  embed_fwd_kernel<<<nblk(rows, 4), 256, 0, s>>>(idx_in, idx_saved, wte, wpe, x, T, C, Vp, rows,
                                                 err);
  return hipGetLastError();
}

hipError_t launch_embed_bwd(const int32_t* idx, const float* dx, float* dwte, float* dwpe, int B,
                            int T, int C, hipStream_t s) {
  long rows = (long)B * T;
  embed_bwd_wte_kernel<<<nblk(rows, 4), 256, 0, s>>>(idx, dx, dwte, C, rows);
  embed_bwd_wpe_kernel<<<nblk((long)T * C, 256), 256, 0, s>>>(dx, dwpe, B, T, C);
  return hipGetLastError();
}

hipError_t launch_layernorm_fwd(DType out_t, const float* x, const float* w, const float* b,
                                void* y, float* mean, float* rstd, long rows, int C,
                                hipStream_t s) {
  if (out_t == DT_BF16)
    layernorm_fwd_kernel<bf16_t><<<nblk(rows, 4), 256, 0, s>>>(x, w, b, (bf16_t*)y, mean, rstd,
                                                               rows, C);
  else
    layernorm_fwd_kernel<float><<<nblk(rows, 4), 256, 0, s>>>(x, w, b, (float*)y, mean, rstd,
                                                              rows, C);
  return hipGetLastError();
}

int ln_bwd_blocks(long rows) { return (int)((rows + LN_BWD_ROWS - 1) / LN_BWD_ROWS); }

hipError_t launch_layernorm_bwd(DType copy_t, const float* dy, const float* x, const float* mean,
                                const float* rstd, const float* w, float* dres, void* dres_copy,
                                int accumulate, float* partial, float* dw, float* db, long rows,
                                int C, hipStream_t s) {
  int nb = ln_bwd_blocks(rows);
  size_t shm = (size_t)8 * C * sizeof(float);
  if (copy_t == DT_BF16)
    layernorm_bwd_kernel<bf16_t><<<nb, 256, shm, s>>>(dy, x, mean, rstd, w, dres,
                                                       (bf16_t*)dres_copy, accumulate, partial,
                                                       rows, C, LN_BWD_ROWS);
  else
    layernorm_bwd_kernel<float><<<nb, 256, shm, s>>>(dy, x, mean, rstd, w, dres,
                                                      (float*)dres_copy, accumulate, partial, rows,
                                                      C, LN_BWD_ROWS);
  colsum_partials_kernel<<<nblk(2 * C, 256), 256, 0, s>>>(partial, nb, 2 * C, dw, db, C);
  return hipGetLastError();
}

hipError_t launch_bias_grad(DType in_t, const void* X, long rows, int N, long ldx, float* partial,
                            float* db, hipStream_t s) {
  int splits = BIAS_SPLITS;
  long rps = (rows + splits - 1) / splits;
  dim3 grid(nblk(N, 256), splits);
  if (in_t == DT_BF16)
    colsum_kernel<bf16_t><<<grid, 256, 0, s>>>((const bf16_t*)X, rows, N, ldx, partial, rps);
  else
    colsum_kernel<float><<<grid, 256, 0, s>>>((const float*)X, rows, N, ldx, partial, rps);
  colsum_partials_kernel<<<nblk(N, 256), 256, 0, s>>>(partial, splits, N, db, db, N);
  return hipGetLastError();
}

hipError_t launch_xent(DType t, void* logits, const int32_t* targets, int* n_valid,
                       float* row_loss, float* loss, long rows, int Vp, int* err, hipStream_t s) {
  count_valid_kernel<<<1, 1024, 0, s>>>(targets, rows, Vp, n_valid, err);
  if (t == DT_BF16) {
    if (Vp > 256 * 8 * 25) return hipErrorInvalidValue;
    xent_fused_kernel<bf16_t, 25><<<(unsigned)rows, 256, 0, s>>>((bf16_t*)logits, targets,
                                                                  n_valid, row_loss, Vp);
  } else {
    if (Vp > 256 * 8 * 25) return hipErrorInvalidValue;
    if (Vp <= 256 * 8 * 4)
      xent_fused_kernel<float, 4><<<(unsigned)rows, 256, 0, s>>>((float*)logits, targets,
                                                                  n_valid, row_loss, Vp);
    else
      xent_fused_kernel<float, 25><<<(unsigned)rows, 256, 0, s>>>((float*)logits, targets,
                                                                   n_valid, row_loss, Vp);
  }
  loss_reduce_kernel<<<1, 1024, 0, s>>>(row_loss, rows, n_valid, loss);
  return hipGetLastError();
}

hipError_t launch_grad_norm(const float* g, long n, double* partial, float max_norm,
                            float* norm_out, float* clip_out, hipStream_t s) {
  sumsq_kernel<<<NORM_PARTS, 256, 0, s>>>(g, n / 4, partial);
  norm_finish_kernel<<<1, 256, 0, s>>>(partial, NORM_PARTS, max_norm, norm_out, clip_out);
  return hipGetLastError();
}

hipError_t launch_adamw(const AdamChunk* chunks, int nchunks, float* p, const float* g, float* m,
                        float* v, bf16_t* shadow, const float* clip, float lr, float b1, float b2,
                        float eps, float wd, float step_size, float inv_sqrt_bc2, hipStream_t s) {
  adamw_kernel<<<nchunks, 256, 0, s>>>(chunks, p, g, m, v, shadow, clip, lr, b1, b2, eps, wd,
                                       step_size, inv_sqrt_bc2);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, long n, float val, hipStream_t s) {
  long blocks = (n / 4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  fill_kernel<<<(unsigned)blocks, 256, 0, s>>>(p, n, val);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* src, bf16_t* dst, long n, hipStream_t s) {
  long blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  f32_to_bf16_kernel<<<(unsigned)(blocks < 1 ? 1 : blocks), 256, 0, s>>>(src, dst, n);
  return hipGetLastError();
}

hipError_t launch_bf16_to_f32(const bf16_t* src, float* dst, long n, hipStream_t s) {
  long blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  bf16_to_f32_kernel<<<(unsigned)(blocks < 1 ? 1 : blocks), 256, 0, s>>>(src, dst, n);
  return hipGetLastError();
}
