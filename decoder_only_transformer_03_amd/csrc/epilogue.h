// GEMM epilogues: what happens to a finished fp32 accumulator C[m][n].
// Every epilogue handles four consecutive columns n..n+3 of one row m.
#pragma once
#include "common.h"

enum EpiKind : int {
  EPI_STORE = 0,     // out[m][n] = alpha*c                                   (out: TO)
  EPI_BIAS_GELU = 1, // h = c + bias[n]; out[m][n] = gelu'(h); out2[m][n] = gelu(h)  (TO)
  EPI_RESID = 2,     // out[m][n] = resid[m][n] + c + bias[n]                  (out, resid: fp32)
  EPI_ACCUM = 3,     // out[m][n] += alpha*c            one writer per element (out: fp32)
  EPI_ATOMIC = 4,    // atomically out[m][n] += alpha*c  split-K               (out: fp32)
  EPI_GELU_BWD = 5,  // out[m][n] = alpha*c * aux[m][n], aux = gelu'(h)          (out, aux: TO)
                     // (+ column sums of the fp32 result into colsum, if set)
  EPI_PARTIAL = 6,   // split-K slice z: out[z*split_stride + m*ldo + n] = alpha*c  (fp32)
  EPI_BIAS = 7,      // out[m][n] = alpha*c + bias[n]                         (out: TO)
  // Fused lm_head + cross-entropy (c = a logit; column n is vocabulary entry col0 + n):
  EPI_LSE = 8,       // per row m and 64-column block b = n/64: (max, sum exp(c - max)) over
                     // the block into part[2 (m*nblk + b) + 0, 1]; tlogit[m] = c at the
                     // target's column                                       (fp32)
  EPI_DLOGITS = 9,   // out[m][n] = (exp(c - lse[m]) - [col0 + n == tgt[m]]) / n_valid,
                     // 0 for rows whose target is -1                        (out: TO)
};

struct EpiArgs {
  void* out;
  long ldo;
  void* out2;
  const float* bias;
  const float* resid;
  long ldr;
  const void* aux;
  long ldx;
  float alpha;
  long split_stride;
  float* colsum;  // EPI_GELU_BWD: [row block of 128][N] partial column sums, or null
  // EPI_LSE / EPI_DLOGITS
  const int32_t* tgt;   // target per row, -1 = no target
  const float* lse;     // log-sum-exp per row (EPI_DLOGITS)
  float* part;          // block partials, 2 floats per (row, 64-column block) (EPI_LSE)
  float* tlogit;        // logit of the target per row (EPI_LSE)
  const int* n_valid;   // rows with a target (EPI_DLOGITS)
  long col0;            // vocabulary index of output column 0
  int nblk;             // 64-column blocks per row of part (EPI_LSE)
};

// d(mean cross-entropy)/d(logit) of one element: softmax - onehot, times
// `scale` (1/n_valid for a row with a target, else 0).
__device__ __forceinline__ float dlogit(float c, float lse, bool is_target, float scale) {
  return (__expf(c - lse) - (is_target ? 1.0f : 0.0f)) * scale;
}
__device__ __forceinline__ float dlogit_scale(const EpiArgs& e, int t) {
  const int nv = *e.n_valid;
  return t != -1 && nv > 0 ? 1.0f / (float)nv : 0.f;
}

// Does the epilogue read memory per element (residual, old value, aux)?
constexpr bool epi_reads(int EPI) {
  return EPI == EPI_RESID || EPI == EPI_ACCUM || EPI == EPI_GELU_BWD;
}
constexpr bool epi_bias(int EPI) {
  return EPI == EPI_BIAS || EPI == EPI_BIAS_GELU || EPI == EPI_RESID;
}

// Phase 1: the per-element input of the epilogue (issue these for a whole
// block of outputs before any store, so the loads overlap).
template <int EPI, typename TO>
__device__ __forceinline__ void epi_load4(const EpiArgs& e, long m, int n, float in[4]) {
  if constexpr (EPI == EPI_RESID) {
    ld4(e.resid + m * e.ldr + n, in);
  } else if constexpr (EPI == EPI_ACCUM) {
    ld4(reinterpret_cast<const float*>(e.out) + m * e.ldo + n, in);
  } else if constexpr (EPI == EPI_GELU_BWD) {
    ld4(reinterpret_cast<const TO*>(e.aux) + m * e.ldx + n, in);
  }
}

__device__ __forceinline__ void epi_load_bias(const EpiArgs& e, int n, float b[4]) {
  if (e.bias) {
    ld4(e.bias + n, b);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = 0.f;
  }
}

// Phase 2: combine accumulator c, input `in` and bias `b`, and store.
template <int EPI, typename TO>
__device__ __forceinline__ void epi_store4(const EpiArgs& e, long m, int n, const float c[4],
                                           const float in[4], const float b[4], int split) {
  float r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = e.alpha * c[j];
  if constexpr (epi_bias(EPI)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] += b[j];
  }
  if constexpr (EPI == EPI_STORE || EPI == EPI_BIAS) {
    st4(reinterpret_cast<TO*>(e.out) + m * e.ldo + n, r);
  } else if constexpr (EPI == EPI_BIAS_GELU) {
    float g[4], d[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) g[j] = gelu_tanh_and_grad_f(r[j], d + j);
    st4(reinterpret_cast<TO*>(e.out) + m * e.ldo + n, d);
    st4(reinterpret_cast<TO*>(e.out2) + m * e.ldo + n, g);
  } else if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] += in[j];
    st4(reinterpret_cast<float*>(e.out) + m * e.ldo + n, r);
  } else if constexpr (EPI == EPI_ACCUM) {
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] += in[j];
    st4(reinterpret_cast<float*>(e.out) + m * e.ldo + n, r);
  } else if constexpr (EPI == EPI_ATOMIC) {
    float* o = reinterpret_cast<float*>(e.out) + m * e.ldo + n;
#pragma unroll
    for (int j = 0; j < 4; ++j) atomicAdd(o + j, r[j]);
  } else if constexpr (EPI == EPI_PARTIAL) {
    st4(reinterpret_cast<float*>(e.out) + split * e.split_stride + m * e.ldo + n, r);
  } else if constexpr (EPI == EPI_GELU_BWD) {
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] *= in[j];
    st4(reinterpret_cast<TO*>(e.out) + m * e.ldo + n, r);
  } else if constexpr (EPI == EPI_DLOGITS) {
    const int t = e.tgt[m];
    const float l = e.lse[m], sc = dlogit_scale(e, t);
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = dlogit(r[j], l, e.col0 + n + j == t, sc);
    st4(reinterpret_cast<TO*>(e.out) + m * e.ldo + n, r);
  }
}

// Both phases for one group of four columns (split: the split-K slice).
template <int EPI, typename TO>
__device__ __forceinline__ void epi_apply4(const EpiArgs& e, long m, int n, const float c[4],
                                           int split) {
  float in[4] = {0.f, 0.f, 0.f, 0.f}, b[4];
  epi_load4<EPI, TO>(e, m, n, in);
  epi_load_bias(e, n, b);
  epi_store4<EPI, TO>(e, m, n, c, in, b, split);
}
