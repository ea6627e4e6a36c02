// Bandwidth-bound kernels of the GPT-2 step: embedding gather / scatter-add,
// LayerNorm forward / backward, fused softmax cross-entropy, bias-gradient
// column sums, global gradient norm and AdamW.  All are row- or
// element-parallel with wavefront (64-lane) reductions and 16-byte accesses.
#include "kernels.h"

// Non-temporal 16-byte load and store (streams used once per kernel).
typedef float nt_f4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 nt_ld4(const float* p) {
  const nt_f4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_f4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void nt_ld4(const float* p, float v[4]) {
  const nt_f4 u = __builtin_nontemporal_load(reinterpret_cast<const nt_f4*>(p));
  v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
}
__device__ __forceinline__ void nt_st4(float* p, const float v[4]) {
  nt_f4 u = {v[0], v[1], v[2], v[3]};
  __builtin_nontemporal_store(u, reinterpret_cast<nt_f4*>(p));
}
__device__ __forceinline__ void nt_st4(float* p, float a, float b, float c, float d) {
  nt_f4 v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<nt_f4*>(p));
}
typedef uint32_t nt_u4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 nt_ldu4(const void* p) {
  const nt_u4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void nt_stu4(void* p, uint4 u) {
  nt_u4 v = {u.x, u.y, u.z, u.w};
  __builtin_nontemporal_store(v, reinterpret_cast<nt_u4*>(p));
}


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
// Deterministic, no atomics, in three launches:
//  1. a stable sort of the positions by token id (one workgroup, radix sort);
//  2. per chunk of EMB_CHUNK sorted positions, the sum of each run of equal
//     ids in position order: a run wholly inside the chunk is added to its
//     dwte row directly (its only writer); the piece of a run that continues
//     into the next chunk (head) and the piece that continues from the
//     previous one (tail) go to per-chunk slots instead;
//  3. per head: head + the following chunks' tails of the same id, in chunk
//     order, added to the dwte row.
constexpr int EMB_CHUNK = 32;
constexpr int SORT_THREADS = 1024;

// Exclusive prefix sum over the workgroup (NTH threads) of v, and the total.
template <int NTH>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum,
                                                         uint32_t* total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (t == 0) {
    uint32_t run = 0;
    for (int i = 0; i < NTH / 64; ++i) {
      const uint32_t c = wsum[i];
      wsum[i] = run;
      run += c;
    }
    wsum[NTH / 64] = run;
  }
  __syncthreads();
  const uint32_t r = wsum[w] + x - v;
  *total = wsum[NTH / 64];
  __syncthreads();
  return r;
}

// Stable LSD radix sort (4-bit digits, npass passes, npass even) of n keys
// (token ids) with their positions as values, over global ping-pong buffers;
// the result is in (ka, va).  Thread t owns a contiguous range of elements:
// it counts their digits, a workgroup scan over the (digit, thread) counters
// gives its output offsets, and it scatters them in their original order.
__global__ __launch_bounds__(SORT_THREADS) void id_sort_kernel(const int32_t* __restrict__ idx,
                                                               long n, int npass,
                                                               uint32_t* __restrict__ ka,
                                                               uint32_t* __restrict__ va,
                                                               uint32_t* __restrict__ kb,
                                                               uint32_t* __restrict__ vb) {
  __shared__ uint32_t cnt[16 * SORT_THREADS];  // [digit][thread]
  __shared__ uint32_t wsum[SORT_THREADS / 64 + 1];
  const int t = threadIdx.x;
  const long per = (n + SORT_THREADS - 1) / SORT_THREADS;
  const long e0 = t * per < n ? t * per : n, e1 = e0 + per < n ? e0 + per : n;
  for (long i = t; i < n; i += SORT_THREADS) {
    ka[i] = (uint32_t)idx[i];
    va[i] = (uint32_t)i;
  }
  __syncthreads();
  uint32_t *ks = ka, *vs = va, *kd = kb, *vd = vb;
  for (int pass = 0; pass < npass; ++pass) {
    const int shift = 4 * pass;
#pragma unroll
    for (int d = 0; d < 16; ++d) cnt[d * SORT_THREADS + t] = 0;
    for (long i = e0; i < e1; ++i) atomicAdd(&cnt[((ks[i] >> shift) & 15u) * SORT_THREADS + t], 1u);
    __syncthreads();
    // exclusive scan over the flattened counters, 16 consecutive per thread
    uint32_t loc[16], sum = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      loc[j] = sum;
      sum += cnt[16 * t + j];
    }
    uint32_t total;
    const uint32_t base = block_exclusive_scan<SORT_THREADS>(sum, wsum, &total);
#pragma unroll
    for (int j = 0; j < 16; ++j) cnt[16 * t + j] = base + loc[j];
    __syncthreads();
    for (long i = e0; i < e1; ++i) {
      const uint32_t k = ks[i];
      const uint32_t o = atomicAdd(&cnt[((k >> shift) & 15u) * SORT_THREADS + t], 1u);
      kd[o] = k;
      vd[o] = vs[i];
    }
    __syncthreads();  // scattered keys visible to the whole workgroup
    uint32_t* tk = ks; ks = kd; kd = tk;
    uint32_t* tv = vs; vs = vd; vd = tv;
    __syncthreads();
  }
}

// The same sort held in LDS, for n <= SORT_LDS_N positions and ids below
// 2^16: each element is packed as id << 16 | position, so sorting by the top
// 16 bits carries the position along.  8-bit digits, so one or two passes.
// Wavefront w owns the contiguous chunk [w*chunk, (w+1)*chunk) and walks it
// 64 elements at a time, lane l taking element s0 + l.  The lanes holding
// the same digit are found with eight ballots (one per digit bit); a lane's
// rank among them is the number of such lanes below it, and the lowest of
// them (rank 0) advances the wavefront's running offset for that digit.
// Counting (LDS atomic adds: the count does not depend on their order) fills
// cnt[w][digit]; the workgroup turns the counts into output offsets
// (digits in order, within a digit the wavefronts in order); the scatter
// walks the chunk again in the same order, so equal ids keep their order.
// The sorted ids and positions go to (ka, va).
constexpr int SORT_LDS_N = 16384;
constexpr int SORT_LDS_THREADS = 1024;
constexpr int SORT_LDS_WAVES = SORT_LDS_THREADS / 64;

// Lanes (among the active ones) whose digit equals this lane's.
__device__ __forceinline__ uint64_t same_digit_lanes(uint32_t d, bool active) {
  uint64_t m = __ballot(active);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (d >> b) & 1u;
    const uint64_t set = __ballot(bit);
    m &= bit ? set : ~set;
  }
  return m;
}

__global__ __launch_bounds__(SORT_LDS_THREADS) void id_sort_lds_kernel(
    const int32_t* __restrict__ idx, int n, int npass, uint32_t* __restrict__ ka,
    uint32_t* __restrict__ va) {
  __shared__ uint32_t buf[2][SORT_LDS_N];
  __shared__ uint32_t cnt[SORT_LDS_WAVES][256];  // per wavefront and digit
  __shared__ uint32_t dbase[256];                // first output slot of each digit
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const uint64_t below = (1ull << lane) - 1;
  const int chunk = (n + SORT_LDS_WAVES - 1) / SORT_LDS_WAVES;
  const int c0 = w * chunk, c1 = c0 + chunk < n ? c0 + chunk : n;  // (empty when c0 >= n)
  // (fixed trip count, so that the loads are issued together)
#pragma unroll
  for (int j = 0; j < SORT_LDS_N / SORT_LDS_THREADS; ++j) {
    const int i = j * SORT_LDS_THREADS + t;
    if (i < n) buf[0][i] = ((uint32_t)idx[i] << 16) | (uint32_t)i;
  }
  __syncthreads();
  int src = 0;
  for (int pass = 0; pass < npass; ++pass) {
    const int shift = 16 + 8 * pass;
    const uint32_t* ks = buf[src];
    uint32_t* kd = buf[src ^ 1];
    // (this wavefront's own row: its later accesses follow in order)
    for (int d = lane; d < 256; d += 64) cnt[w][d] = 0;
    for (int i = c0 + lane; i < c1; i += 64) atomicAdd(&cnt[w][(ks[i] >> shift) & 255u], 1u);
    __syncthreads();
    if (t < 256) {  // per digit: exclusive prefix over the wavefronts, and the total
      uint32_t run = 0;
      for (int v = 0; v < SORT_LDS_WAVES; ++v) {
        const uint32_t c = cnt[v][t];
        cnt[v][t] = run;
        run += c;
      }
      dbase[t] = run;
    }
    __syncthreads();
    if (w == 0) {  // exclusive prefix of the digit totals, four digits per lane
      uint32_t v[4], own = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = dbase[4 * lane + j];
        own += v[j];
      }
      uint32_t inc = own;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = __shfl_up(inc, o, 64);
        if (lane >= o) inc += u;
      }
      uint32_t run = inc - own;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dbase[4 * lane + j] = run;
        run += v[j];
      }
    }
    __syncthreads();
    for (int s0 = c0; s0 < c1; s0 += 64) {
      const bool act = s0 + lane < c1;
      const uint32_t k = act ? ks[s0 + lane] : 0u;
      const uint32_t d = (k >> shift) & 255u;
      const uint64_t m = same_digit_lanes(d, act);
      const uint32_t rank = (uint32_t)__popcll(m & below);
      // every lane reads its digit's running offset before the lowest lane of
      // the digit advances it (one wavefront: LDS accesses in program order)
      const uint32_t o = dbase[d] + cnt[w][d] + rank;
      if (act) kd[o] = k;
      if (act && rank == 0) cnt[w][d] += (uint32_t)__popcll(m);
    }
    __syncthreads();
    src ^= 1;
  }
#pragma unroll
  for (int j = 0; j < SORT_LDS_N / SORT_LDS_THREADS; ++j) {
    const int i = j * SORT_LDS_THREADS + t;
    if (i < n) {
      const uint32_t k = buf[src][i];
      ka[i] = k >> 16;
      va[i] = k & 0xffffu;
    }
  }
}

// Step 2: one workgroup per chunk of EMB_CHUNK sorted positions (keys = ids,
// vals = positions); thread t sums columns 4t.. (stride 1024).  head/tail:
// [chunk][C] slots; hflag/tflag[chunk]: the id of the chunk's head / tail
// piece, or -1.
__global__ __launch_bounds__(256) void embed_bwd_chunk_kernel(const uint32_t* __restrict__ keys,
                                                              const uint32_t* __restrict__ vals,
                                                              const float* __restrict__ dx,
                                                              float* __restrict__ dwte,
                                                              float* __restrict__ head,
                                                              float* __restrict__ tail,
                                                              int* __restrict__ hflag,
                                                              int* __restrict__ tflag, int C,
                                                              long n) {
  __shared__ uint32_t key[EMB_CHUNK], pos[EMB_CHUNK];
  const long p0 = (long)blockIdx.x * EMB_CHUNK;
  const int m = n - p0 < EMB_CHUNK ? (int)(n - p0) : EMB_CHUNK;
  const int t = threadIdx.x;
  if (t < m) {
    key[t] = keys[p0 + t];
    pos[t] = vals[p0 + t];
  }
  __syncthreads();
  // does the first run continue from the previous chunk, the last into the next?
  const bool cont_in = p0 > 0 && keys[p0 - 1] == key[0];
  const bool cont_out = p0 + m < n && keys[p0 + m] == key[m - 1];
  if (t == 0) {
    tflag[blockIdx.x] = cont_in ? (int)key[0] : -1;
    // a chunk inside one run has no head of its own: the run started earlier
    const bool one_run = key[0] == key[m - 1];
    hflag[blockIdx.x] = cont_out && !(one_run && cont_in) ? (int)key[m - 1] : -1;
  }
  // Run ending at position q: it continues a run from the previous chunk when
  // it is the chunk's first run (keys are sorted, so its key is key[0]) and
  // cont_in; it goes on into the next chunk when q is the last position and
  // cont_out; otherwise it lies wholly here and is added into its dwte row.
  // The runs of a chunk have distinct ids, so a batch's dwte rows are loaded
  // before any of its stores: one round trip per batch, not one per run.
  auto run_end = [&](int q) { return q + 1 == m || key[q + 1] != key[q]; };
  auto from_prev = [&](int q) { return cont_in && key[q] == key[0]; };
  auto to_next = [&](int q) { return q + 1 == m && cont_out; };
  for (int c = t * 4; c < C; c += 1024) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int q0 = 0; q0 < m; q0 += 8) {
      float4 v[8], o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)  // issue the batch's loads before using any
        if (q0 + j < m) v[j] = *reinterpret_cast<const float4*>(dx + (long)pos[q0 + j] * C + c);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = q0 + j;
        if (q < m && run_end(q) && !from_prev(q) && !to_next(q))
          o[j] = *reinterpret_cast<const float4*>(dwte + (long)key[q] * C + c);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = q0 + j;
        if (q >= m) break;
        acc.x += v[j].x; acc.y += v[j].y; acc.z += v[j].z; acc.w += v[j].w;
        if (run_end(q)) {
          if (from_prev(q)) {         // continues a run
            *reinterpret_cast<float4*>(tail + (long)blockIdx.x * C + c) = acc;
          } else if (to_next(q)) {    // run goes on
            *reinterpret_cast<float4*>(head + (long)blockIdx.x * C + c) = acc;
          } else {                    // whole run here
            float4 r = o[j];
            r.x += acc.x; r.y += acc.y; r.z += acc.z; r.w += acc.w;
            *reinterpret_cast<float4*>(dwte + (long)key[q] * C + c) = r;
          }
          acc = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
  }
}

// Step 3: one workgroup per chunk with a head: head + tails of the following
// chunks while they continue the same id, in chunk order, into the dwte row.
// The run's last chunk is found first (all threads test one flag each), so
// that the tails' loads can be issued in batches.
__global__ __launch_bounds__(256) void embed_bwd_fix_kernel(const float* __restrict__ head,
                                                            const float* __restrict__ tail,
                                                            const int* __restrict__ hflag,
                                                            const int* __restrict__ tflag,
                                                            float* __restrict__ dwte, int C,
                                                            int nchunks) {
  __shared__ int stop;
  const int ch = blockIdx.x;
  const int id = hflag[ch];
  if (id < 0) return;
  // end = first chunk after ch that does not continue the run
  int end = ch + 1;
  for (;;) {
    if (threadIdx.x == 0) stop = nchunks;
    __syncthreads();
    const int k = end + (int)threadIdx.x;
    if (k < nchunks && tflag[k] != id) atomicMin(&stop, k);
    __syncthreads();
    const int st = stop;
    __syncthreads();
    if (st < nchunks || end + 256 >= nchunks) {
      end = st < end + 256 ? st : (end + 256 < nchunks ? end + 256 : nchunks);
      break;
    }
    end += 256;
  }
  for (int c = threadIdx.x * 4; c < C; c += 1024) {
    float4 a = *reinterpret_cast<const float4*>(head + (long)ch * C + c);
    for (int k0 = ch + 1; k0 < end; k0 += 8) {
      float4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (k0 + j < end) v[j] = *reinterpret_cast<const float4*>(tail + (long)(k0 + j) * C + c);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (k0 + j < end) {
          a.x += v[j].x; a.y += v[j].y; a.z += v[j].z; a.w += v[j].w;
        }
    }
    float* d = dwte + (long)id * C + c;
    float4 o = *reinterpret_cast<const float4*>(d);
    o.x += a.x; o.y += a.y; o.z += a.z; o.w += a.w;
    *reinterpret_cast<float4*>(d) = o;
  }
}

// dwpe[t,c] += sum_b dx[b,t,c], or = with store   (deterministic: one thread
// per (t, c))
__global__ __launch_bounds__(256) void embed_bwd_wpe_kernel(const float* __restrict__ dx,
                                                            float* __restrict__ dwpe, int B, int T,
                                                            int C, int store) {
  long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)T * C) return;
  const float* p = dx + i;
  const long st = (long)T * C;
  float s = 0.f;
  int b = 0;
  for (; b + 8 <= B; b += 8) {  // eight loads in flight, added in order of b
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(long)(b + u) * st];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; b < B; ++b) s += p[(long)b * st];
  dwpe[i] = store ? s : dwpe[i] + s;
}

// ---------------------------------------------------------------------------
// LayerNorm forward: y = (x - mean) * rstd * w + b, rstd = 1/sqrt(var + 1e-5),
// biased variance over C.  One wavefront per LN_FWD_RPW rows, kept in
// registers: their loads (and the weight and bias loads) are all in flight
// before the first reduction.
// ---------------------------------------------------------------------------
constexpr int LN_MAXV = 8;  // float4 per lane: C <= 2048
// rows per wavefront: at B*T = 16384, C = 768, one row (4096 workgroups) is
// 5% faster than two and four
constexpr int LN_FWD_RPW = 1;

template <int NV, typename TO>
__global__ __launch_bounds__(256) void layernorm_fwd_kernel(const float* __restrict__ x,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ b,
                                                            TO* __restrict__ y,
                                                            float* __restrict__ mean_out,
                                                            float* __restrict__ rstd_out,
                                                            long rows, int C) {
  const long row0 = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * LN_FWD_RPW;
  const int lane = threadIdx.x & 63;
  if (row0 >= rows) return;
  float v[LN_FWD_RPW][NV][4], g[NV][4], bb[NV][4];
#pragma unroll
  for (int r = 0; r < LN_FWD_RPW; ++r) {
    if (row0 + r >= rows) break;
    const float* xr = x + (row0 + r) * C;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = (i * 64 + lane) * 4;
      if (c < C) nt_ld4(xr + c, v[r][i]);  // read again only in the backward
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = (i * 64 + lane) * 4;
    if (c < C) {
      ld4(w + c, g[i]);
      ld4(b + c, bb[i]);
    }
  }
#pragma unroll
  for (int r = 0; r < LN_FWD_RPW; ++r) {
    const long row = row0 + r;
    if (row >= rows) break;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if ((i * 64 + lane) * 4 < C) s += (v[r][i][0] + v[r][i][1]) + (v[r][i][2] + v[r][i][3]);
    const float mean = wave_sum(s) / (float)C;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if ((i * 64 + lane) * 4 < C) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float d = v[r][i][j] - mean;
          q += d * d;
        }
      }
    }
    const float var = wave_sum(q) / (float)C;
    const float rstd = 1.0f / sqrtf(var + 1e-5f);
    TO* yr = y + row * C;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = (i * 64 + lane) * 4;
      if (c < C) {
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = (v[r][i][j] - mean) * rstd * g[i][j] + bb[i][j];
        st4(yr + c, o);
      }
    }
    if (lane == 0) {
      mean_out[row] = mean;
      rstd_out[row] = rstd;
    }
  }
}

// ---------------------------------------------------------------------------
// LayerNorm backward.  With xhat = (x - mean) rstd and d = dy * w:
//   dx = rstd (d - mean(d) - xhat mean(d xhat)),  dw = sum dy xhat, db = sum dy.
// dres = dx (accumulate = 0) or dres += dx; an optional bf16 copy of the new
// dres feeds the next bf16 GEMM.  Per-workgroup partial column sums of
// [dw | db | new dres] (the last is the bias gradient of the linear layer
// that consumes dres) go to partial[blockIdx.x][3C].
// ---------------------------------------------------------------------------
template <int NV, typename TB>
__global__ __launch_bounds__(256) void layernorm_bwd_kernel(
    const float* __restrict__ dy, const float* __restrict__ x, const float* __restrict__ mean,
    const float* __restrict__ rstd, const float* __restrict__ w, float* __restrict__ dres,
    TB* __restrict__ dres_copy, int accumulate, float* __restrict__ partial, long rows, int C,
    int rows_per_block) {
  extern __shared__ float sred[];  // [4][3C]
  int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float dg[NV][4], db[NV][4], ds[NV][4], wv[NV][4];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int c = (i * 64 + lane) * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) dg[i][j] = db[i][j] = ds[i][j] = 0.f;
    if (c < C) ld4(w + c, wv[i]);
  }
  long r0 = (long)blockIdx.x * rows_per_block;
  long r1 = r0 + rows_per_block < rows ? r0 + rows_per_block : rows;
  // two rows per wavefront at a time (row, row + 4): all their loads -- dy,
  // x and the old dres -- are issued before any reduction needs them
  for (long row0 = r0 + wave; row0 < r1; row0 += 8) {
    float g[2][NV][4], xh[2][NV][4], o[2][NV][4], mu[2], rs[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const long row = row0 + 4 * q;
      const bool on = row < r1;
      mu[q] = on ? mean[row] : 0.f;
      rs[q] = on ? rstd[row] : 0.f;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        int c = (i * 64 + lane) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) g[q][i][j] = xh[q][i][j] = o[q][i][j] = 0.f;
        if (on && c < C) {
          ld4(dy + row * C + c, g[q][i]);
          ld4(x + row * C + c, xh[q][i]);
          if (accumulate) ld4(dres + row * C + c, o[q][i]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const long row = row0 + 4 * q;
      if (row >= r1) break;
      float s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        int c = (i * 64 + lane) * 4;
        if (c < C) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float gg = g[q][i][j];
            const float xhat = (xh[q][i][j] - mu[q]) * rs[q];
            xh[q][i][j] = xhat;
            dg[i][j] += gg * xhat;
            db[i][j] += gg;
            const float d = gg * wv[i][j];
            g[q][i][j] = d;
            s1 += d;
            s2 += d * xhat;
          }
        }
      }
      s1 = wave_sum(s1) / (float)C;
      s2 = wave_sum(s2) / (float)C;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        int c = (i * 64 + lane) * 4;
        if (c < C) {
          float* ov = o[q][i];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float dx = rs[q] * (g[q][i][j] - s1 - xh[q][i][j] * s2);
            ov[j] = accumulate ? ov[j] + dx : dx;
            ds[i][j] += ov[j];
          }
          st4(dres + row * C + c, ov);
          if (dres_copy) st4(dres_copy + row * C + c, ov);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int c = (i * 64 + lane) * 4;
    if (c < C) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sred[wave * 3 * C + c + j] = dg[i][j];
        sred[wave * 3 * C + C + c + j] = db[i][j];
        sred[wave * 3 * C + 2 * C + c + j] = ds[i][j];
      }
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < 3 * C; c += 256) {
    float t = (sred[c] + sred[3 * C + c]) + (sred[6 * C + c] + sred[9 * C + c]);
    partial[(long)blockIdx.x * 3 * C + c] = t;
  }
}

// Column sums of a (rows x N) matrix: workgroup (64 columns) x (rows of one
// split), 4 row phases per workgroup, fixed summation order.
// partial[split][n] = sum over the split's rows.
template <typename T>
__global__ __launch_bounds__(256) void colsum_kernel(const T* __restrict__ X, long rows, int N,
                                                     long ldx, float* __restrict__ partial,
                                                     long rows_per_split) {
  __shared__ float s[4][64];
  const int c = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int n = blockIdx.x * 64 + c;
  const long r0 = (long)blockIdx.y * rows_per_split;
  const long r1 = r0 + rows_per_split < rows ? r0 + rows_per_split : rows;
  float a = 0.f;
  if (n < N) {
    long r = r0 + g;
    for (; r + 12 < r1; r += 16)
      a += (ldf(X + r * ldx + n) + ldf(X + (r + 4) * ldx + n)) +
           (ldf(X + (r + 8) * ldx + n) + ldf(X + (r + 12) * ldx + n));
    for (; r < r1; r += 4) a += ldf(X + r * ldx + n);
  }
  s[g][c] = a;
  __syncthreads();
  if (g == 0 && n < N) partial[(long)blockIdx.y * N + n] = (s[0][c] + s[1][c]) + (s[2][c] + s[3][c]);
}

// Column sums of every listed partial-sum matrix, one launch: a workgroup per
// 64-column chunk of one problem (found by binary search over the problems'
// first chunks), four row phases per column with four accumulators each, in a
// fixed order.  dst[k][j] += sum over the parts of column k*w + j.
__global__ __launch_bounds__(256) void colsum_grouped_kernel(const ColsumProblem* __restrict__ probs,
                                                             int nprobs, long M, int nblk,
                                                             int store) {
  __shared__ float sh[4][64];
  int lo = 0, hi = nprobs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (probs[mid].chunk0 <= (int)blockIdx.x) lo = mid;
    else hi = mid - 1;
  }
  const ColsumProblem& P = probs[lo];
  const int ncols = P.ncols;
  const long nparts = P.rows_per_part > 0   ? (M + P.rows_per_part - 1) / P.rows_per_part
                      : P.rows_per_part < 0 ? (long)nblk
                                            : (long)P.fixed_parts;
  const int cl = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int c = ((int)blockIdx.x - P.chunk0) * 64 + cl;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  if (c < ncols) {
    const float* p = P.partial + c;
    long r = g;
    for (; r + 12 < nparts; r += 16) {
      a0 += p[r * ncols];
      a1 += p[(r + 4) * ncols];
      a2 += p[(r + 8) * ncols];
      a3 += p[(r + 12) * ncols];
    }
    for (; r < nparts; r += 4) a0 += p[r * ncols];
  }
  sh[g][cl] = (a0 + a1) + (a2 + a3);
  __syncthreads();
  if (g != 0 || c >= ncols) return;
  const int k = c / P.w, j = c - k * P.w;
  float* d = P.dst[k];
  if (d) {
    const float v = (sh[0][cl] + sh[1][cl]) + (sh[2][cl] + sh[3][cl]);
    d[j] = store ? v : d[j] + v;
  }
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
  for (long i0 = threadIdx.x; i0 < rows; i0 += 8 * 1024) {  // eight loads in flight
    int t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = i0 + 1024L * u < rows ? tgt[i0 + 1024L * u] : -1;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (t[u] != -1) {
        ++cnt;
        if (t[u] < 0 || t[u] >= Vp) bad = 1;
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
  // opaque to the optimiser: values derived from r before this are not reused
  __device__ void touch() { asm volatile("" : "+v"(r.x), "+v"(r.y), "+v"(r.z), "+v"(r.w)); }
  __device__ void load(const bf16_t* p) { r = nt_ldu4(p); }
  __device__ float get(int j) const {
    uint32_t w = j < 2 ? r.x : j < 4 ? r.y : j < 6 ? r.z : r.w;
    return (j & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
  __device__ static void store(bf16_t* p, const float v[8]) {
    nt_stu4(p, make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]),
                          pack_bf2(v[6], v[7])));
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


// One workgroup per row.  The row is read from memory once into registers
// (XENT_KPT chunks of 8 per thread), reduced to its maximum and sum of
// exponentials over the workgroup, and overwritten with
//   d(loss)/d(logits) = (softmax - onehot(target)) / n_valid   (0 if ignored).
// Padded vocabulary columns take part like real ones.
// The exponentials run on exp2 with the scalings folded into one fma per
// element: exp(x - M) = 2^(x log2e - M log2e), and softmax / n_valid =
// 2^(x log2e - (lse log2e + log2 n_valid)).  Only the thread that holds the
// target's chunk forms (softmax - 1) / n_valid, for that one element.
// 1024 threads of 7 chunks: 4.5% faster than 512 of 13 on the 50304-wide rows
// (768 of 9: 2%; 256 of 25: 15% slower).
constexpr int XENT_NT = 1024, XENT_KPT = 7;  // rows up to 8 * 1024 * 7 = 57344 wide
constexpr float XENT_LOG2E = 1.4426950408889634f;
template <typename T, bool GRAD>
__global__ __launch_bounds__(XENT_NT) void xent_fused_kernel(T* __restrict__ logits,
                                                             const int32_t* __restrict__ targets,
                                                             const int* __restrict__ n_valid,
                                                             float* __restrict__ row_loss, int Vp) {
  constexpr int NW = XENT_NT / 64;
  __shared__ float red[2][NW];
  const long row = blockIdx.x;
  T* lr = logits + row * (long)Vp;
  int tgt = targets[row];
  const bool valid = tgt != -1;
  if (tgt < 0 || tgt >= Vp) tgt = -1;  // out-of-range already flagged by count_valid
  const float xt = valid && tgt >= 0 ? ldf(lr + tgt) : 0.f;
  const int nchunks = Vp >> 3, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nv = *n_valid;
  if (GRAD && !(valid && nv > 0)) {
    // an ignored position (or none valid): its row of d(logits) is zero
    float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < XENT_KPT; ++i) {
      const int ch = threadIdx.x + i * XENT_NT;
      if (ch < nchunks) Row8<T>::store(lr + ch * 8, z);
    }
    if (threadIdx.x == 0) row_loss[row] = 0.f;
    return;
  }
  Row8<T> v[XENT_KPT];
#pragma unroll
  for (int i = 0; i < XENT_KPT; ++i) {
    const int ch = threadIdx.x + i * XENT_NT;
    if (ch < nchunks) v[i].load(lr + ch * 8);
  }
  float m = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < XENT_KPT; ++i)
    if (threadIdx.x + i * XENT_NT < nchunks)
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, v[i].get(j));
  m = wave_max(m);
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < XENT_KPT; ++i) v[i].touch();
  }
  if (lane == 0) red[0][w] = m;
  __syncthreads();
  float M = red[0][0];
#pragma unroll
  for (int i = 1; i < NW; ++i) M = fmaxf(M, red[0][i]);
  const float mb = -M * XENT_LOG2E;
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < XENT_KPT; ++i)
    if (threadIdx.x + i * XENT_NT < nchunks)
#pragma unroll
      for (int j = 0; j < 8; ++j) sum += __builtin_amdgcn_exp2f(fmaf(v[i].get(j), XENT_LOG2E, mb));
  sum = wave_sum(sum);
  if constexpr (sizeof(T) == 2) {
    // keep only the packed row live across the reduction (the float copies
    // would double the registers and halve the blocks per CU)
#pragma unroll
    for (int i = 0; i < XENT_KPT; ++i) v[i].touch();
  }
  if (lane == 0) red[1][w] = sum;
  __syncthreads();
  float S = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) S += red[1][i];
  const float lse = M + __logf(S);
  if constexpr (GRAD) {
    const float scale = 1.0f / (float)nv;
    const float pb = -(lse * XENT_LOG2E + __log2f((float)nv));
    // the chunk offsets are recomputed here from an opaque copy of the thread
    // index instead of being kept live since the loads: fewer registers, so
    // more rows share a CU
    int tx = (int)threadIdx.x;
    asm volatile("" : "+v"(tx));
#pragma unroll
    for (int i = 0; i < XENT_KPT; ++i) {
      const int ch = tx + i * XENT_NT;
      if (ch < nchunks) {
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = __builtin_amdgcn_exp2f(fmaf(v[i].get(j), XENT_LOG2E, pb));
        Row8<T>::store(lr + ch * 8, o);
      }
    }
    // the target's element, rewritten by the thread that stored its chunk
    // (its two stores reach memory in program order)
    if (tgt >= 0 && (tgt >> 3) % XENT_NT == (int)threadIdx.x)
      stf(lr + tgt, (__expf(xt - lse) - 1.0f) * scale);
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
  for (long i0 = threadIdx.x; i0 < rows; i0 += 8 * 1024) {  // eight loads in flight, same order
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = i0 + 1024L * u < rows ? row_loss[i0 + 1024L * u] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) a += (double)v[u];
  }
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

// Fused lm_head loss, one wavefront per row: the row's log-sum-exp from the
// (max m_b, sum s_b of exp(logit - m_b)) partials of its 64-column blocks,
//   lse = M + log(sum_b s_b exp(m_b - M)),  M = max_b m_b,
// and row_loss = lse - logit[target] (0 without a target; an out-of-range
// target, flagged by count_valid, counts its logit as 0).
__global__ __launch_bounds__(256) void head_lse_kernel(const float* __restrict__ part, int nblk,
                                                       const float* __restrict__ tlogit,
                                                       const int32_t* __restrict__ targets,
                                                       long rows, int Vp, float* __restrict__ lse,
                                                       float* __restrict__ row_loss) {
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float2* p = reinterpret_cast<const float2*>(part) + row * nblk;
  float mx = -__builtin_inff();
  for (int b = lane; b < nblk; b += 64) mx = fmaxf(mx, p[b].x);
  mx = wave_max(mx);
  float sum = 0.f;
  for (int b = lane; b < nblk; b += 64) {
    const float2 q = p[b];
    sum += q.y * __expf(q.x - mx);
  }
  sum = wave_sum(sum);
  if (lane == 0) {
    const float l = mx + __logf(sum);
    const int t = targets[row];
    const float xt = t >= 0 && t < Vp ? tlogit[row] : 0.f;
    lse[row] = l;
    row_loss[row] = t != -1 ? l - xt : 0.f;
  }
}

// Per-sequence mean loss over the positions with a target:
// seq_loss[b] = sum_t row_loss[b*T + t] / #{t : targets[b*T + t] != -1}, 0 if none.
// One workgroup per sequence; fp64 sum in a fixed order.
__global__ __launch_bounds__(256) void seq_loss_kernel(const float* __restrict__ row_loss,
                                                       const int32_t* __restrict__ targets,
                                                       int T, float* __restrict__ seq_loss) {
  __shared__ double s[4];
  __shared__ int c[4];
  const long r0 = (long)blockIdx.x * T;
  double a = 0.0;
  int n = 0;
  for (int t = threadIdx.x; t < T; t += 256) {
    a += (double)row_loss[r0 + t];
    n += targets[r0 + t] != -1;
  }
  a = wave_sum_d(a);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o, 64);
  if ((threadIdx.x & 63) == 0) {
    s[threadIdx.x >> 6] = a;
    c[threadIdx.x >> 6] = n;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const double t = (s[0] + s[1]) + (s[2] + s[3]);
    const int nn = (c[0] + c[1]) + (c[2] + c[3]);
    seq_loss[blockIdx.x] = nn > 0 ? (float)(t / nn) : 0.f;
  }
}

hipError_t launch_seq_loss(const float* row_loss, const int32_t* targets, int B, int T,
                           float* seq_loss, hipStream_t s) {
  seq_loss_kernel<<<B, 256, 0, s>>>(row_loss, targets, T, seq_loss);
  return hipGetLastError();
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
  const long stride = (long)gridDim.x * 256;
  long i = (long)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n4; i += 4 * stride) {  // four loads in flight
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = nt_ld4(g + 4 * (i + u * stride));
#pragma unroll
    for (int u = 0; u < 4; ++u)
      a += (double)v[u].x * v[u].x + (double)v[u].y * v[u].y + (double)v[u].z * v[u].z +
           (double)v[u].w * v[u].w;
  }
  for (; i < n4; i += stride) {
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
  int n4 = ck.len >> 2;
#pragma unroll 4
  for (int i = threadIdx.x; i < n4; i += 256) {
    const float4 pp = nt_ld4(p + ck.start + 4L * i), gg = nt_ld4(g + ck.start + 4L * i);
    const float4 mm = nt_ld4(m + ck.start + 4L * i), vv = nt_ld4(v + ck.start + 4L * i);
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
    nt_st4(p + ck.start + 4L * i, P[0], P[1], P[2], P[3]);
    nt_st4(m + ck.start + 4L * i, M[0], M[1], M[2], M[3]);
    nt_st4(v + ck.start + 4L * i, V[0], V[1], V[2], V[3]);
    if (shadow) st4(shadow + ck.start + 4 * (long)i, P);
  }
}

// AdamW on 64 x 64 tiles of the decayed matrices that the input-gradient
// products also read transposed: the same update as adamw_kernel, and besides
// the bf16 copy at the same offset, its transpose (cols x rows) into
// shadow_t, through LDS.  Each load or store instruction of a wavefront
// covers four whole 64-element rows (16 lanes x 4 elements per row): lane l
// of wavefront w takes rows 16w + 4q + l/16 (q = 0..3), columns 4 (l%16) ..
// +3; the transposed tile is written the same way.
__global__ __launch_bounds__(256) void adamw_tiles_kernel(const TTile* __restrict__ tiles,
                                                          float* __restrict__ p,
                                                          const float* __restrict__ g,
                                                          float* __restrict__ m,
                                                          float* __restrict__ v,
                                                          bf16_t* __restrict__ shadow,
                                                          bf16_t* __restrict__ shadow_t,
                                                          const float* __restrict__ clip, float lr,
                                                          float b1, float b2, float eps, float wd,
                                                          float step_size, float inv_sqrt_bc2) {
  __shared__ uint16_t t[64][66];  // padded rows: the column reads spread over the banks
  const TTile tt = tiles[blockIdx.x];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c4 = 4 * (l & 15);
  const float c = *clip;
  const float decay = 1.0f - lr * wd;
  const long tile0 = tt.off + (long)tt.r0 * tt.cols + tt.c0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 16 * w + 4 * q + (l >> 4);
    const long e = tile0 + (long)r * tt.cols + c4;
    // streamed once per step, far larger than the caches: non-temporal
    const float4 pp = nt_ld4(p + e), gg = nt_ld4(g + e), mm = nt_ld4(m + e), vv = nt_ld4(v + e);
    float P[4] = {pp.x, pp.y, pp.z, pp.w}, G[4] = {gg.x, gg.y, gg.z, gg.w};
    float M[4] = {mm.x, mm.y, mm.z, mm.w}, V[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float gj = G[j] * c;
      P[j] *= decay;
      M[j] = b1 * M[j] + (1.0f - b1) * gj;
      V[j] = b2 * V[j] + (1.0f - b2) * gj * gj;
      P[j] -= step_size * M[j] / (sqrtf(V[j]) * inv_sqrt_bc2 + eps);
    }
    nt_st4(p + e, P[0], P[1], P[2], P[3]);
    nt_st4(m + e, M[0], M[1], M[2], M[3]);
    nt_st4(v + e, V[0], V[1], V[2], V[3]);
    const uint32_t w0 = pack_bf2(P[0], P[1]), w1 = pack_bf2(P[2], P[3]);
    *reinterpret_cast<uint2*>(shadow + e) = make_uint2(w0, w1);
    t[r][c4] = (uint16_t)(w0 & 0xffffu);
    t[r][c4 + 1] = (uint16_t)(w0 >> 16);
    t[r][c4 + 2] = (uint16_t)(w1 & 0xffffu);
    t[r][c4 + 3] = (uint16_t)(w1 >> 16);
  }
  __syncthreads();
  // row oc of the transpose = column oc of the tile; this lane's 4 tile rows
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int oc = 16 * w + 4 * q + (l >> 4);
    const uint32_t o0 = (uint32_t)t[c4][oc] | ((uint32_t)t[c4 + 1][oc] << 16);
    const uint32_t o1 = (uint32_t)t[c4 + 2][oc] | ((uint32_t)t[c4 + 3][oc] << 16);
    *reinterpret_cast<uint2*>(shadow_t + tt.off + (long)(tt.c0 + oc) * tt.rows + tt.r0 + c4) =
        make_uint2(o0, o1);
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

size_t embed_bwd_scratch_bytes(long rows, int C) {
  const long nch = (rows + EMB_CHUNK - 1) / EMB_CHUNK;
  return (size_t)4 * rows * sizeof(uint32_t) + (size_t)2 * nch * C * sizeof(float) +
         (size_t)2 * nch * sizeof(int) + 256;
}

hipError_t launch_embed_bwd(const int32_t* idx, const float* dx, float* dwte, float* dwpe, int B,
                            int T, int C, int Vp, void* scratch, bool wpe_store, hipStream_t s) {
  const long rows = (long)B * T;
  const long nch = (rows + EMB_CHUNK - 1) / EMB_CHUNK;
  if (C % 4) return hipErrorInvalidValue;
  uint32_t* ka = reinterpret_cast<uint32_t*>(scratch);
  uint32_t* va = ka + rows;
  uint32_t* kb = va + rows;
  uint32_t* vb = kb + rows;
  float* head = reinterpret_cast<float*>(vb + rows);
  float* tail = head + nch * C;
  int* hflag = reinterpret_cast<int*>(tail + nch * C);
  int* tflag = hflag + nch;
  int bits = 1;
  while (bits < 31 && (1L << bits) < (long)Vp) ++bits;
  if (rows <= SORT_LDS_N && bits <= 16) {
    id_sort_lds_kernel<<<1, SORT_LDS_THREADS, 0, s>>>(idx, (int)rows, (bits + 7) / 8, ka, va);
  } else {
    int npass = (bits + 3) / 4;
    npass += npass & 1;  // even: the sorted result ends in (ka, va)
    id_sort_kernel<<<1, SORT_THREADS, 0, s>>>(idx, rows, npass, ka, va, kb, vb);
  }
  embed_bwd_chunk_kernel<<<(unsigned)nch, 256, 0, s>>>(ka, va, dx, dwte, head, tail, hflag, tflag,
                                                       C, rows);
  embed_bwd_fix_kernel<<<(unsigned)nch, 256, 0, s>>>(head, tail, hflag, tflag, dwte, C, (int)nch);
  embed_bwd_wpe_kernel<<<nblk((long)T * C, 256), 256, 0, s>>>(dx, dwpe, B, T, C, wpe_store ? 1 : 0);
  return hipGetLastError();
}

template <int NV>
static void ln_fwd_nv(DType out_t, const float* x, const float* w, const float* b, void* y,
                      float* mean, float* rstd, long rows, int C, hipStream_t s) {
  if (out_t == DT_BF16)
    layernorm_fwd_kernel<NV, bf16_t><<<nblk(rows, 4 * LN_FWD_RPW), 256, 0, s>>>(
        x, w, b, (bf16_t*)y, mean, rstd, rows, C);
  else
    layernorm_fwd_kernel<NV, float><<<nblk(rows, 4 * LN_FWD_RPW), 256, 0, s>>>(
        x, w, b, (float*)y, mean, rstd, rows, C);
}

hipError_t launch_layernorm_fwd(DType out_t, const float* x, const float* w, const float* b,
                                void* y, float* mean, float* rstd, long rows, int C,
                                hipStream_t s) {
  switch ((C + 255) / 256) {
    case 1: ln_fwd_nv<1>(out_t, x, w, b, y, mean, rstd, rows, C, s); break;
    case 2: ln_fwd_nv<2>(out_t, x, w, b, y, mean, rstd, rows, C, s); break;
    case 3: ln_fwd_nv<3>(out_t, x, w, b, y, mean, rstd, rows, C, s); break;
    case 4: ln_fwd_nv<4>(out_t, x, w, b, y, mean, rstd, rows, C, s); break;
    case 5: ln_fwd_nv<5>(out_t, x, w, b, y, mean, rstd, rows, C, s); break;
    case 6: ln_fwd_nv<6>(out_t, x, w, b, y, mean, rstd, rows, C, s); break;
    case 7: ln_fwd_nv<7>(out_t, x, w, b, y, mean, rstd, rows, C, s); break;
    case 8: ln_fwd_nv<8>(out_t, x, w, b, y, mean, rstd, rows, C, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int ln_bwd_blocks(long rows) { return (int)((rows + LN_BWD_ROWS - 1) / LN_BWD_ROWS); }

template <int NV>
static hipError_t ln_bwd_nv(DType copy_t, const float* dy, const float* x, const float* mean,
                            const float* rstd, const float* w, float* dres, void* dres_copy,
                            int accumulate, float* partial, long rows, int C, int nb, size_t shm,
                            hipStream_t s) {
  if (shm > 65536) {  // wide models: allow more than the default dynamic LDS
    hipError_t e = copy_t == DT_BF16
        ? hipFuncSetAttribute((const void*)layernorm_bwd_kernel<NV, bf16_t>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm)
        : hipFuncSetAttribute((const void*)layernorm_bwd_kernel<NV, float>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
  }
  if (copy_t == DT_BF16)
    layernorm_bwd_kernel<NV, bf16_t><<<nb, 256, shm, s>>>(dy, x, mean, rstd, w, dres,
                                                           (bf16_t*)dres_copy, accumulate, partial,
                                                           rows, C, LN_BWD_ROWS);
  else
    layernorm_bwd_kernel<NV, float><<<nb, 256, shm, s>>>(dy, x, mean, rstd, w, dres,
                                                          (float*)dres_copy, accumulate, partial,
                                                          rows, C, LN_BWD_ROWS);
  return hipGetLastError();
}

hipError_t launch_layernorm_bwd(DType copy_t, const float* dy, const float* x, const float* mean,
                                const float* rstd, const float* w, float* dres, void* dres_copy,
                                int accumulate, float* partial, long rows, int C, hipStream_t s) {
  int nb = ln_bwd_blocks(rows);
  size_t shm = (size_t)12 * C * sizeof(float);
  hipError_t e;
  switch ((C + 255) / 256) {
#define LNB(NV) \
  case NV: e = ln_bwd_nv<NV>(copy_t, dy, x, mean, rstd, w, dres, dres_copy, accumulate, partial, rows, C, nb, shm, s); break;
    LNB(1) LNB(2) LNB(3) LNB(4) LNB(5) LNB(6) LNB(7) LNB(8)
#undef LNB
    default: return hipErrorInvalidValue;
  }
  return e;
}

hipError_t launch_colsum_grouped(const ColsumProblem* d_probs, int nprobs, int total_chunks, long M,
                                 int nblk, bool store, hipStream_t s) {
  if (nprobs <= 0 || total_chunks <= 0) return hipSuccess;
  colsum_grouped_kernel<<<total_chunks, 256, 0, s>>>(d_probs, nprobs, M, nblk, store ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_colsum_parts(DType in_t, const void* X, long rows, int N, long ldx, float* partial,
                               hipStream_t s) {
  int splits = BIAS_SPLITS;
  long rps = (rows + splits - 1) / splits;
  dim3 grid(nblk(N, 64), splits);
  if (in_t == DT_BF16)
    colsum_kernel<bf16_t><<<grid, 256, 0, s>>>((const bf16_t*)X, rows, N, ldx, partial, rps);
  else
    colsum_kernel<float><<<grid, 256, 0, s>>>((const float*)X, rows, N, ldx, partial, rps);
  return hipGetLastError();
}

hipError_t launch_xent(DType t, void* logits, const int32_t* targets, int* n_valid,
                       float* row_loss, float* loss, long rows, int Vp, int* err, bool grad,
                       hipStream_t s) {
  if (Vp % 8 || Vp > 8 * XENT_NT * XENT_KPT) return hipErrorInvalidValue;
  count_valid_kernel<<<1, 1024, 0, s>>>(targets, rows, Vp, n_valid, err);
  if (t == DT_BF16)
    grad ? xent_fused_kernel<bf16_t, true><<<(unsigned)rows, XENT_NT, 0, s>>>(
               (bf16_t*)logits, targets, n_valid, row_loss, Vp)
         : xent_fused_kernel<bf16_t, false><<<(unsigned)rows, XENT_NT, 0, s>>>(
               (bf16_t*)logits, targets, n_valid, row_loss, Vp);
  else
    grad ? xent_fused_kernel<float, true><<<(unsigned)rows, XENT_NT, 0, s>>>(
               (float*)logits, targets, n_valid, row_loss, Vp)
         : xent_fused_kernel<float, false><<<(unsigned)rows, XENT_NT, 0, s>>>(
               (float*)logits, targets, n_valid, row_loss, Vp);
  loss_reduce_kernel<<<1, 1024, 0, s>>>(row_loss, rows, n_valid, loss);
  return hipGetLastError();
}

// Transposed copy of 64 x 64 bf16 tiles through LDS: 256 threads, each
// moving two 8-element row pieces in and two 8-element column pieces out.
__global__ __launch_bounds__(256) void transpose_tiles_kernel(const bf16_t* __restrict__ src,
                                                              bf16_t* __restrict__ dst,
                                                              const TTile* __restrict__ tiles) {
  __shared__ uint16_t t[64][66];  // padded rows: column reads spread over the banks
  const TTile tt = tiles[blockIdx.x];
  const int tid = threadIdx.x, q = tid & 7;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = (tid >> 3) + 32 * h;
    const uint4 v = *reinterpret_cast<const uint4*>(src + tt.off + (long)(tt.r0 + r) * tt.cols +
                                                    tt.c0 + 8 * q);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      t[r][8 * q + 2 * j] = (uint16_t)(w[j] & 0xffffu);
      t[r][8 * q + 2 * j + 1] = (uint16_t)(w[j] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = (tid >> 3) + 32 * h;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)t[8 * q + 2 * j][c] | ((uint32_t)t[8 * q + 2 * j + 1][c] << 16);
    *reinterpret_cast<uint4*>(dst + tt.off + (long)(tt.c0 + c) * tt.rows + tt.r0 + 8 * q) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

hipError_t launch_transpose_tiles(const bf16_t* src, bf16_t* dst, const TTile* tiles, int ntiles,
                                  hipStream_t s) {
  if (ntiles <= 0) return hipSuccess;
  transpose_tiles_kernel<<<(unsigned)ntiles, 256, 0, s>>>(src, dst, tiles);
  return hipGetLastError();
}

hipError_t launch_head_loss(const float* part, int nblk, const float* tlogit,
                           const int32_t* targets, int* n_valid, float* lse, float* row_loss,
                           float* loss, long rows, int Vp, int* err, hipStream_t s) {
  count_valid_kernel<<<1, 1024, 0, s>>>(targets, rows, Vp, n_valid, err);
  head_lse_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(part, nblk, tlogit, targets, rows,
                                                             Vp, lse, row_loss);
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

hipError_t launch_adamw_tiles(const TTile* tiles, int ntiles, float* p, const float* g, float* m,
                              float* v, bf16_t* shadow, bf16_t* shadow_t, const float* clip,
                              float lr, float b1, float b2, float eps, float wd, float step_size,
                              float inv_sqrt_bc2, hipStream_t s) {
  if (ntiles <= 0) return hipSuccess;
  adamw_tiles_kernel<<<(unsigned)ntiles, 256, 0, s>>>(tiles, p, g, m, v, shadow, shadow_t, clip,
                                                      lr, b1, b2, eps, wd, step_size,
                                                      inv_sqrt_bc2);
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

