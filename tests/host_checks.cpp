// Host-side checks of libgpt2's runtime, built with the host compiler's
// address and undefined-behaviour sanitizers and run without a GPU: every
// entry point's argument and shape checks, and for valid configurations the
// whole host plan that gpt2_init builds before its first device call (the
// workspace layout, the AdamW chunk and tile tables, the grouped
// weight-gradient and column-sum problem tables).  With no device that
// first call fails, so gpt2_init must return GPT2_E_HIP and leave *out NULL
// (with a device it returns GPT2_OK and nothing runs on it here).  Exit
// status 0 when every expectation holds; a sanitizer report aborts.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include <hip/hip_runtime.h>

#include "../include/gpt2.h"
#include "../include/gpt2_ops.h"

static int failures = 0;
#define EXPECT(cond)                                                      \
  do {                                                                    \
    if (!(cond)) {                                                        \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

static gpt2_config cfg(int L, int H, int C, int V, int Vp, int bs, int mb, int prec, int hc) {
  gpt2_config c;
  c.n_layer = L;
  c.n_head = H;
  c.n_embd = C;
  c.vocab_size = V;
  c.padded_vocab_size = Vp;
  c.block_size = bs;
  c.max_batch = mb;
  c.precision = prec;
  c.head_chunk = hc;
  return c;
}

int main() {
  // with a device present, gpt2_init would send its tables to the fake
  // workspace address below: these checks are for hosts without one
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    std::printf("a device is present: skipped\n");
    return 77;
  }
  // valid configurations: tiny fp32, bf16 shapes of 124M and XL width,
  // ragged capacities, fused heads
  std::vector<gpt2_config> good = {
      cfg(2, 4, 128, 512, 512, 64, 4, GPT2_FP32, 0),
      cfg(2, 4, 128, 512, 512, 64, 300, GPT2_FP32, 192),
      cfg(2, 2, 128, 512, 512, 1000, 9, GPT2_BF16, 0),
      cfg(12, 12, 768, 50257, 50304, 1024, 16, GPT2_BF16, 0),
      cfg(12, 12, 768, 50257, 50304, 1024, 3, GPT2_BF16, 4096),
      cfg(2, 25, 1600, 50257, 50304, 1024, 8, GPT2_BF16, 0),
      cfg(1, 1, 64, 1, 64, 1, 1, GPT2_BF16, 64),
  };
  // the fake workspace is never dereferenced on the host
  void* fake = reinterpret_cast<void*>(uintptr_t(1) << 40);
  for (const gpt2_config& c : good) {
    const size_t n = gpt2_num_params(&c);
    EXPECT(n > 0);
    size_t bytes = 0;
    EXPECT(gpt2_workspace_bytes(&c, &bytes) == GPT2_OK);
    EXPECT(bytes > 4 * sizeof(float) * n);
    gpt2_t* h = reinterpret_cast<gpt2_t*>(1);
    const gpt2_status st = gpt2_init(&c, fake, bytes, nullptr, 42, &h);
    EXPECT(st == GPT2_E_HIP || st == GPT2_OK);
    if (st == GPT2_OK) {
      gpt2_destroy(h);
    } else {
      EXPECT(h == nullptr);
    }
    // too small a workspace, misaligned, NULL
    EXPECT(gpt2_init(&c, fake, bytes - 1, nullptr, 1, &h) == GPT2_E_ARG && h == nullptr);
    EXPECT(gpt2_init(&c, reinterpret_cast<char*>(fake) + 16, bytes, nullptr, 1, &h) == GPT2_E_ARG);
    EXPECT(gpt2_init(&c, nullptr, bytes, nullptr, 1, &h) == GPT2_E_ARG);
    EXPECT(gpt2_init(&c, fake, bytes, nullptr, 1, nullptr) == GPT2_E_ARG);
  }
  // invalid configurations
  std::vector<gpt2_config> bad = {
      cfg(12, 7, 768, 50257, 50304, 1024, 2, GPT2_BF16, 0),    // C % H
      cfg(12, 24, 768, 50257, 50304, 1024, 2, GPT2_BF16, 0),   // bf16 head width 32
      cfg(12, 12, 768, 50257, 50257, 1024, 2, GPT2_BF16, 0),   // Vp % 64
      cfg(12, 12, 768, 50257, 50240, 1024, 2, GPT2_BF16, 0),   // Vp < V
      cfg(12, 64, 4096, 50257, 50304, 1024, 2, GPT2_BF16, 0),  // C too wide
      cfg(12, 12, 768, 50257, 50304, 0, 2, GPT2_BF16, 0),      // block_size
      cfg(2, 4, 128, 512, 512, 64, 0, GPT2_FP32, 0),           // max_batch
      cfg(2, 4, 128, 512, 512, 64, 4, 7, 0),                   // precision
      cfg(2, 4, 128, 512, 512, 64, 4, GPT2_FP32, 100),         // head_chunk % 64
      cfg(0, 4, 128, 512, 512, 64, 4, GPT2_FP32, 0),           // n_layer
  };
  for (const gpt2_config& c : bad) {
    EXPECT(gpt2_num_params(&c) == 0);
    size_t bytes = 0;
    EXPECT(gpt2_workspace_bytes(&c, &bytes) == GPT2_E_ARG);
    gpt2_t* h = nullptr;
    EXPECT(gpt2_init(&c, fake, size_t(1) << 40, nullptr, 1, &h) == GPT2_E_ARG && h == nullptr);
  }
  EXPECT(gpt2_num_params(nullptr) == 0);
  EXPECT(gpt2_workspace_bytes(nullptr, nullptr) == GPT2_E_ARG);
  // learning-rate schedule: the section's fixed points, its argument checks
  double lr = -1.0;
  EXPECT(gpt2_lr_at(715, 6e-4, 6e-5, 715, 19073, &lr) == GPT2_OK && std::fabs(lr - 6e-4) < 1e-18);
  EXPECT(gpt2_lr_at(19073, 6e-4, 6e-5, 715, 19073, &lr) == GPT2_OK && std::fabs(lr - 6e-5) < 1e-15);
  EXPECT(gpt2_lr_at(0, 6e-4, 6e-5, 715, 19073, &lr) == GPT2_OK && std::fabs(lr - 6e-4 / 715) < 1e-18);
  for (int64_t t = 0; t < 25000; t += 37) EXPECT(gpt2_lr_at(t, 6e-4, 6e-5, 715, 19073, &lr) == GPT2_OK);
  EXPECT(gpt2_lr_at(-1, 6e-4, 6e-5, 715, 19073, &lr) == GPT2_E_ARG);
  EXPECT(gpt2_lr_at(0, 6e-4, 6e-5, 0, 10, &lr) == GPT2_E_ARG);
  EXPECT(gpt2_lr_at(0, 6e-4, 6e-5, 10, 5, &lr) == GPT2_E_ARG);
  EXPECT(gpt2_lr_at(0, 6e-4, 6e-5, 10, 20, nullptr) == GPT2_E_ARG);
  // calls on a NULL handle
  float f = 0.f;
  int64_t i64 = 0;
  EXPECT(gpt2_set_params(nullptr, &f, 1, 0) == GPT2_E_ARG);
  EXPECT(gpt2_get(nullptr, GPT2_PARAMS, &f, 1, 0) == GPT2_E_ARG);
  EXPECT(gpt2_set_state(nullptr, GPT2_GRADS, &f, 1, 0) == GPT2_E_ARG);
  EXPECT(gpt2_get_step(nullptr, &i64) == GPT2_E_ARG);
  EXPECT(gpt2_set_step(nullptr, 1) == GPT2_E_ARG);
  EXPECT(gpt2_forward(nullptr, nullptr, nullptr, 1, 1, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_eval(nullptr, nullptr, nullptr, 1, 1, nullptr, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_forward_last(nullptr, nullptr, 1, 1, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_sample(nullptr, nullptr, 4, 1, 1, 1.f, 0, nullptr, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_generate(nullptr, nullptr, 1, 1, 1, 1.f, 0, nullptr, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_generate_cached(nullptr, nullptr, 1, 1, 1, 1.f, 0, nullptr, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_prefill(nullptr, nullptr, 1, 1, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_decode(nullptr, nullptr, 1, 1, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_get_loss(nullptr, &f) == GPT2_E_ARG);
  EXPECT(gpt2_zero_grad(nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_backward(nullptr, 1.f) == GPT2_E_ARG);
  EXPECT(gpt2_adamw_step(nullptr, 1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.f, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_get_grad_norm(nullptr, &f) == GPT2_E_ARG);
  EXPECT(gpt2_sync(nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_get_activation(nullptr, GPT2_ACT_LNF, 0, &f, 1) == GPT2_E_ARG);
  EXPECT(gpt2_timing_begin(nullptr, 0) == GPT2_E_ARG);
  EXPECT(gpt2_timing_end(nullptr, nullptr, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_wgrad_layout(nullptr, nullptr, nullptr, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_last_error(nullptr) != nullptr);
  gpt2_destroy(nullptr);
  // single-kernel entry points: argument checks before any launch
  EXPECT(gpt2_op_gemm(GPT2_BF16, 4, 4, 4, nullptr, 4, 0, fake, 4, 0, reinterpret_cast<float*>(fake),
                      4, 1.f, 0, 0, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_op_gemm(GPT2_BF16, 4, 4, 4, fake, 4, 1, fake, 4, 0, reinterpret_cast<float*>(fake), 4,
                      1.f, 0, 0, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_op_gemm(7, 4, 4, 4, fake, 4, 0, fake, 4, 0, reinterpret_cast<float*>(fake), 4, 1.f, 0,
                      0, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_op_gemm_epi(8, 64, 64, nullptr, 64, fake, 64, 0, nullptr, nullptr, 0, fake, nullptr,
                          64, GPT2_BF16, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_op_gemm_epi(8, 64, 64, fake, 64, fake, 64, 3, nullptr, nullptr, 0, fake, nullptr, 64,
                          GPT2_BF16, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_op_gemm_epi(8, 64, 64, fake, 64, fake, 64, 1, nullptr, nullptr, 0, fake, nullptr, 64,
                          GPT2_BF16, nullptr) == GPT2_E_ARG);  // GELU needs C2
  EXPECT(gpt2_op_gemm_epi(8, 64, 64, fake, 64, fake, 64, 2, nullptr, nullptr, 0, fake, nullptr, 64,
                          GPT2_FP32, nullptr) == GPT2_E_ARG);  // residual needs R
  EXPECT(gpt2_op_gemm_epi(8, 64, 64, fake, 64, fake, 64, 0, nullptr, nullptr, 0, fake, nullptr, 64,
                          GPT2_FP32, nullptr) == GPT2_E_ARG);  // bias output is bf16
  EXPECT(gpt2_op_attention_fwd(GPT2_BF16, nullptr, fake, reinterpret_cast<float*>(fake), 1, 1, 1,
                               64, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_op_attention_bwd(GPT2_BF16, fake, fake, reinterpret_cast<float*>(fake), fake, fake,
                               nullptr, 1, 1, 1, 64, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_op_attention_bwd_noalloc(GPT2_BF16, fake, fake, reinterpret_cast<float*>(fake), fake,
                                       fake, 1025, 1024, 1, 64, nullptr) == GPT2_E_ARG);
  EXPECT(gpt2_op_attention_bwd_noalloc(GPT2_BF16, fake, nullptr, reinterpret_cast<float*>(fake),
                                       fake, fake, 1, 1, 1, 64, nullptr) == GPT2_E_ARG);
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
