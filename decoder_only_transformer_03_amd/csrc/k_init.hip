// Seeded parameter initialisation on the device ("GPT-2 from Scratch",
// Initialization: 0.02, and the residual scaling).
//
// Element e of the flat parameter vector draws the standard normal number e
// of the seed's stream:
//   counter-based generator Philox4x32 with 10 rounds (Salmon, Moraes, Dror,
//   Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011): block
//   b = e / 4 encrypts the counter (b mod 2^32, b / 2^32, 0, 0) under the
//   key (seed mod 2^32, seed / 2^32) into four 32-bit words x0..x3;
//   uniforms u = (floor(x / 2^9) + 1/2) / 2^23, exact in fp32, in (0, 1);
//   Box-Muller (Box and Muller, 1958) on (x0, x1) and on (x2, x3):
//   r = sqrt(-2 ln u_a), z_a = r cos(2 pi u_b), z_b = r sin(2 pi u_b);
//   element 4b + j takes z_j.
// A weight tensor's element is std * z; the seed alone fixes every value,
// whatever the launch shape.
#include "kernels.h"

namespace {

__device__ __forceinline__ void mulhilo(uint32_t a, uint32_t b, uint32_t& hi, uint32_t& lo) {
  const uint64_t p = (uint64_t)a * b;
  hi = (uint32_t)(p >> 32);
  lo = (uint32_t)p;
}

// Ten rounds of the Philox4x32 bijection: each round multiplies words 0 and 2
// by the two round multipliers, mixes the high halves with words 1 and 3 and
// the round key, and the key advances by the two Weyl increments.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo(0xD2511F53u, c.x, hi0, lo0);
    mulhilo(0xCD9E8D57u, c.z, hi1, lo1);
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

__device__ __forceinline__ float unit_open(uint32_t x) {
  return ((float)(x >> 9) + 0.5f) * 0x1p-23f;
}

__device__ __forceinline__ void box_muller(uint32_t xa, uint32_t xb, float& za, float& zb) {
  const float r = sqrtf(-2.0f * logf(unit_open(xa)));
  float s, c;
  sincospif(2.0f * unit_open(xb), &s, &c);  // 2 u exact: sin, cos of 2 pi u
  za = r * c;
  zb = r * s;
}

// p[i] = std * z(e0 + i) for 0 <= i < n; one thread per block of four
// stream elements overlapping [e0, e0 + n).
__global__ __launch_bounds__(256) void init_normal_kernel(float* __restrict__ p, long n, long e0,
                                                          float std, uint32_t k0, uint32_t k1) {
  const long b = (e0 >> 2) + (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long e_first = b << 2;
  if (e_first >= e0 + n) return;
  const uint4 x = philox4x32_10(make_uint4((uint32_t)b, (uint32_t)((uint64_t)b >> 32), 0u, 0u),
                                k0, k1);
  float z[4];
  box_muller(x.x, x.y, z[0], z[1]);
  box_muller(x.z, x.w, z[2], z[3]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const long e = e_first + j;
    if (e >= e0 && e < e0 + n) p[e - e0] = std * z[j];
  }
}

}  // namespace

hipError_t launch_init_normal(float* p, long n, long e0, float std, uint64_t seed,
                              hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long blocks = ((e0 + n - 1) >> 2) - (e0 >> 2) + 1;
  const long grid = (blocks + 255) / 256;
  init_normal_kernel<<<(unsigned)grid, 256, 0, s>>>(p, n, e0, std, (uint32_t)seed,
                                                     (uint32_t)(seed >> 32));
  return hipGetLastError();
}
