// One multinomial draw per row of logits, after temperature and top-k
// ("GPT-2 from Scratch", A generation loop):
//   x = logits / temperature;
//   top-k: entries below the k-th largest x are dropped (entries equal to it stay);
//   p = softmax(x) over the entries kept;
//   token = the smallest i whose cumulative probability exceeds u, u a
//           caller-supplied uniform in [0, 1) (the draw as an inverse CDF over
//           the vocabulary in index order; if rounding leaves no such i, the
//           last entry kept).
//
// One workgroup of 1024 threads per row.  Thread t keeps the row's entries
// [52t, 52t + 52) in registers for the whole kernel: the k-th largest value is
// found exactly by a 4-pass radix select on order-preserving integer keys
// (LDS histograms of 256 bins) over the entries at or above the k-th largest
// of the threads' maxima (found the same way first), gathered in LDS; the sum
// of exponentials and its prefix over threads are fixed-order reductions,
// and the thread whose prefix interval holds u * sum walks its own entries
// to the draw.
#include <type_traits>

#include "kernels.h"

namespace {

constexpr int SMP_NT = 1024, SMP_PER = 52;  // rows up to 53248 wide
constexpr int SMP_NW = SMP_NT / 64;

// Larger float -> larger unsigned key (finite values and -inf).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__global__ __launch_bounds__(SMP_NT) void sample_kernel(const float* __restrict__ logits, long ld,
                                                         int V, float temperature, int top_k,
                                                         const float* __restrict__ uni,
                                                         long u_stride, int32_t* __restrict__ out,
                                                         long out_stride) {
  __shared__ uint32_t hist[2][256];    // radix select, by pass parity
  __shared__ uint32_t sel[2][2];       // radix select: chosen bin, k remaining
  __shared__ float red[SMP_NW];
  __shared__ int redi[SMP_NW];
  __shared__ float incl[SMP_NT];       // inclusive prefix of the per-thread sums
  __shared__ int choice;
  __shared__ uint32_t cand[SMP_NT];    // keys at or above the select's lower bound
  __shared__ uint32_t ncand;
  const long row = blockIdx.x;
  const float* lr = logits + row * ld;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int i0 = t * SMP_PER;

  // entries past V are -inf: below every real entry, zero probability
  float x[SMP_PER];
#pragma unroll
  for (int q = 0; q < SMP_PER / 4; ++q) {
    const int i = i0 + 4 * q;
    if (i + 3 < V) {
      const float4 v = *reinterpret_cast<const float4*>(lr + i);
      x[4 * q + 0] = v.x;
      x[4 * q + 1] = v.y;
      x[4 * q + 2] = v.z;
      x[4 * q + 3] = v.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) x[4 * q + j] = i + j < V ? lr[i + j] : -__builtin_inff();
    }
  }
  if (temperature != 1.0f) {  // x / 1 is x
#pragma unroll
    for (int j = 0; j < SMP_PER; ++j) x[j] = x[j] / temperature;
  }

  // maximum of this thread's entries (as a key: the lower bound below)
  float tmx = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < SMP_PER; ++j) tmx = fmaxf(tmx, x[j]);

  // Exact k-th largest of the counted keys (k of them at least): most
  // significant byte first, each pass keeps the bin where the count from the
  // top reaches the k still wanted.  key_of(j) gives this thread's key j of
  // KEYS, 0 for one that is not counted (every real key is above 0).
  // Two barriers per pass: the histogram and the chosen bin alternate
  // between two buffers by pass parity, and wavefront 0 clears each
  // histogram right after scanning it, for the pass after next.
  if (t < 512) (&hist[0][0])[t] = 0;
  __syncthreads();
  auto kth_key = [&](auto keys_tag, auto key_of, uint32_t k) {
    constexpr int KEYS = decltype(keys_tag)::value;
    uint32_t prefix = 0, pmask = 0, krem = k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass, pb = pass & 1;
      uint32_t* hb = hist[pb];
#pragma unroll
      for (int j = 0; j < KEYS; ++j) {
        const uint32_t key = key_of(j);
        if (key != 0u && (key & pmask) == prefix) atomicAdd(&hb[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (w == 0) {
        // lane l owns bins 255 - 4l .. 252 - 4l (descending); suffix sums
        // from the top by an inclusive scan over the lanes
        uint32_t b[4], own = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          b[j] = hb[255 - 4 * lane - j];
          own += b[j];
        }
        uint32_t inc = own;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t v = __shfl_up(inc, o, 64);
          if (lane >= o) inc += v;
        }
        const uint32_t before = inc - own;
        if (before < krem && inc >= krem) {  // exactly one lane
          uint32_t c = before;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (c + b[j] >= krem) {
              sel[pb][0] = 255u - 4u * lane - j;
              sel[pb][1] = krem - c;
              break;
            }
            c += b[j];
          }
        }
        // cleared for the pass after next (only this wavefront reads it)
#pragma unroll
        for (int j = 0; j < 4; ++j) hb[4 * lane + j] = 0;
      }
      __syncthreads();
      prefix |= sel[pb][0] << shift;
      pmask |= 255u << shift;
      krem = sel[pb][1];
    }
    return prefix;
  };
  using One = std::integral_constant<int, 1>;

  // The k-th largest of the threads' maxima bounds the k-th largest entry
  // from below (k threads hold an entry at least that large).  The entries at
  // or above it -- usually a few times k -- are gathered into LDS, one per
  // thread, and the select runs over them; if there are more than threads,
  // over the entries at or above the bound in place.  Same threshold either
  // way: every entry of the k largest is among those counted.
  uint32_t thr = 0;  // keys >= thr are kept
  if (top_k > 0 && top_k < V) {
    const uint32_t tkey = order_key(tmx);
    const uint32_t lo =
        top_k <= SMP_NT ? kth_key(One{}, [&](int) { return tkey; }, (uint32_t)top_k) : 1u;
    // gather: per entry, the wavefront reserves slots for its lanes at or
    // above the bound with one LDS atomic (slot order does not matter: the
    // select counts)
    if (t == 0) ncand = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SMP_PER; ++j) {
      const uint32_t key = order_key(x[j]);
      const bool c = key >= lo;
      const unsigned long long m = __ballot(c);
      if (m) {
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&ncand, (uint32_t)__popcll(m));
        base = __shfl(base, 0, 64);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (c && base + below < (uint32_t)SMP_NT) cand[base + below] = key;
      }
    }
    __syncthreads();
    const int total = (int)ncand;
    if (total <= SMP_NT) {
      const uint32_t ck = t < total ? cand[t] : 0u;
      thr = kth_key(One{}, [&](int) { return ck; }, (uint32_t)top_k);
    } else {
      thr = kth_key(std::integral_constant<int, SMP_PER>{}, [&](int j) {
        const uint32_t key = order_key(x[j]);
        return key >= lo ? key : 0u;
      }, (uint32_t)top_k);
    }
  }

  // maximum (always kept) and this thread's exponentials
  float mx = wave_max(tmx);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int i = 1; i < SMP_NW; ++i) mx = fmaxf(mx, red[i]);
  float csum = 0.f;
  int last = -1;  // last kept index of this thread
#pragma unroll
  for (int j = 0; j < SMP_PER; ++j) {
    const bool keep = x[j] > -__builtin_inff() && order_key(x[j]) >= thr;
    x[j] = keep ? __expf(x[j] - mx) : 0.f;
    csum += x[j];
    if (keep) last = i0 + j;
  }

  // inclusive prefix of csum over threads: wavefront scans, then the
  // wavefront totals
  float inc = csum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float v = __shfl_up(inc, o, 64);
    if (lane >= o) inc += v;
  }
  __syncthreads();  // red is reused
  if (lane == 63) red[w] = inc;
  int lastw = last;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int v = __shfl_xor(lastw, o, 64);
    lastw = v > lastw ? v : lastw;
  }
  if (lane == 0) redi[w] = lastw;
  __syncthreads();
  float off = 0.f;
  for (int i = 0; i < w; ++i) off += red[i];
  inc += off;
  incl[t] = inc;
  if (t == 0) {
    int l = redi[0];
    for (int i = 1; i < SMP_NW; ++i) l = redi[i] > l ? redi[i] : l;
    choice = l;  // no interval holds the target: the last entry kept
  }
  __syncthreads();
  const float total = incl[SMP_NT - 1];
  const float target = uni[row * u_stride] * total;
  const float lo = t > 0 ? incl[t - 1] : 0.f;
  if (lo <= target && target < inc) {  // at most one thread: the intervals tile [0, total)
    float a = lo;
    int pick = last;
#pragma unroll
    for (int j = 0; j < SMP_PER; ++j) {
      a += x[j];
      if (x[j] > 0.f && a > target) {
        pick = i0 + j;
        break;
      }
    }
    choice = pick;
  }
  __syncthreads();
  if (t == 0) out[row * out_stride] = choice;
}

}  // namespace

hipError_t launch_sample(const float* logits, long ld, int rows, int V, float temperature,
                         int top_k, const float* uni, long u_stride, int32_t* out,
                         long out_stride, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (V < 1 || V > SMP_NT * SMP_PER || ld < V || ld % 4 ||
      reinterpret_cast<uintptr_t>(logits) % 16 || !(temperature > 0.f))
    return hipErrorInvalidValue;
  sample_kernel<<<(unsigned)rows, SMP_NT, 0, s>>>(logits, ld, V, temperature, top_k, uni, u_stride,
                                                  out, out_stride);
  return hipGetLastError();
}
