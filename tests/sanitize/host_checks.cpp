// Host-side checks of the C ABI for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (no GPU: every call here
// returns before any launch). Exits non-zero on the first failed check; the
// sanitizers abort on any memory or undefined-behaviour error they see.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "plp.h"

static int g_fail = 0;

#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      g_fail = 1;                                                    \
    }                                                                \
  } while (0)

static void* fake_device(size_t bytes) {
  // host memory standing in for device pointers: the checks only read the
  // pointer values (NULL-ness and alignment), never the memory
  void* p = nullptr;
  if (posix_memalign(&p, 256, bytes ? bytes : 256) != 0) abort();
  return p;
}

static plp_args base_args(void* h, void* W, void* y, void* m, void* A) {
  plp_args a;
  memset(&a, 0, sizeof(a));
  a.struct_size = sizeof(plp_args);
  a.dtype = PLP_DTYPE_BF16;
  a.B = 2;
  a.T = 64;
  a.H = 256;
  a.V = 1000;
  a.hidden = h;
  a.weight = W;
  a.targets = (const int64_t*)y;
  a.completion_mask = (const uint8_t*)m;
  a.advantages = (const float*)A;
  a.loss_type = PLP_LOSS_GMPO;
  a.is_level = PLP_IS_TOKEN;
  a.reduction = PLP_REDUCE_SEQ_MEAN;
  a.epsilon_low = 0.2;
  a.epsilon_high = 0.2;
  a.temperature = 1.0;
  a.top_entropy_quantile = 1.0;
  return a;
}

int main() {
  CHECK(plp_abi_version() == PLP_ABI_VERSION);
  void* h = fake_device(2 * 64 * 256 * 2);
  void* W = fake_device(1000 * 256 * 2);
  void* y = fake_device(128 * 8);
  void* m = fake_device(128);
  void* A = fake_device(2 * 4);
  void* out_buf = fake_device(1 << 20);
  plp_outputs o;
  memset(&o, 0, sizeof(o));
  o.struct_size = sizeof(o);
  o.loss = (float*)out_buf;
  o.metrics = (float*)out_buf + 64;

  // workspace sizes over many shapes and options (the carving runs with a
  // NULL base)
  const int Hs[] = {64, 96, 128, 256, 384, 896, 1000};
  const int Vs[] = {1, 31, 33, 1000, 151936};
  const int64_t Ts[] = {1, 7, 64, 2048, 32768};
  for (int dt = 0; dt < 2; ++dt)
    for (int H : Hs)
      for (int V : Vs)
        for (int64_t T : Ts)
          for (int q = 0; q < 2; ++q)
            for (int ch = 0; ch < 2; ++ch) {
              plp_args a = base_args(h, W, y, m, A);
              a.dtype = dt;
              a.H = H;
              a.V = V;
              a.B = 3;
              a.T = T;
              a.top_entropy_quantile = q ? 0.2 : 1.0;
              a.chunk_sequences = ch;
              a.bias = (V & 1) ? W : nullptr;
              size_t bytes = 0;
              CHECK(plp_workspace_size(&a, &bytes) == PLP_OK);
              CHECK(bytes > 0 && bytes % 256 == 0);
              // with the caller's matrix-core copy of the weight, less by its size
              size_t wp = 0;
              if (plp_prepared_weight_size(H, V, dt, &wp) == PLP_OK) {
                a.weight_prepared = W;
                size_t bytes2 = 0;
                CHECK(plp_workspace_size(&a, &bytes2) == PLP_OK);
                CHECK(bytes2 + wp == bytes);
              } else {
                a.weight_prepared = W;
                size_t bytes2 = 0;
                CHECK(plp_workspace_size(&a, &bytes2) == PLP_E_UNSUPPORTED);
              }
            }

  // argument errors of the fused call
  {
    plp_args a = base_args(h, W, y, m, A);
    std::vector<char> ws(1 << 16);
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(nullptr, &o, nullptr, 0, nullptr) == PLP_E_INVALID);
    CHECK(strlen(plp_last_error()) > 0);
    a.struct_size = 8;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_INVALID);
    a = base_args(h, W, y, m, A);
    a.B = 0;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_INVALID);
    a = base_args(h, W, y, m, A);
    a.B = (int64_t)1 << 20;
    a.T = (int64_t)1 << 12;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_INVALID);
    a = base_args(h, W, y, m, A);
    a.loss_type = 9;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_INVALID);
    a = base_args(h, W, y, m, A);
    a.is_level = PLP_IS_SEQUENCE;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_UNSUPPORTED);
    a = base_args(h, W, y, m, A);
    a.loss_type = PLP_LOSS_GSPO_TOKEN;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_UNSUPPORTED);
    a = base_args(h, W, y, m, A);
    a.top_entropy_quantile = 1.5;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_INVALID);
    a.top_entropy_quantile = -0.1;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_INVALID);
    a = base_args(h, W, y, m, A);
    a.beta = 0.1;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_INVALID);
    a = base_args(h, W, y, m, A);
    a.temperature = 0.0;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_INVALID);
    a = base_args(h, W, y, m, A);
    a.epsilon_low = -1.0;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_INVALID);
    a = base_args(h, W, y, m, A);
    a.epsilon_high = 0.0 / 0.0;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_INVALID);
    a = base_args(h, W, y, m, A);
    a.chunk_sequences = -1;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_INVALID);
    a = base_args(h, W, y, m, A);
    a.hidden = (const char*)h + 2;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_INVALID);
    a = base_args(h, W, y, m, A);
    a.H = 5000;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_UNSUPPORTED);
    a = base_args(h, W, y, m, A);
    a.token_advantages = (const float*)A;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_UNSUPPORTED);
    a = base_args(h, W, y, m, A);
    a.global_tokens = -3;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_INVALID);
    // outputs
    a = base_args(h, W, y, m, A);
    plp_outputs o2 = o;
    o2.grad_bias = out_buf;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o2, nullptr, 0, nullptr) == PLP_E_INVALID);
    o2 = o;
    o2.loss = nullptr;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o2, nullptr, 0, nullptr) == PLP_E_INVALID);
    o2 = o;
    o2.struct_size = 4;
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o2, nullptr, 0, nullptr) == PLP_E_INVALID);
    // workspace: NULL, too small, misaligned
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, nullptr, 0, nullptr) == PLP_E_WORKSPACE);
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, ws.data(), 100, nullptr) == PLP_E_WORKSPACE);
    size_t need = 0;
    CHECK(plp_workspace_size(&a, &need) == PLP_OK);
    char* big = (char*)fake_device(need + 512);
    CHECK(plp_fused_lmhead_policy_loss_fwd_bwd(&a, &o, big + 16, need, nullptr) == PLP_E_WORKSPACE);
    free(big);
    // an args struct of ABI version 1 (ends before global_tokens) reads the
    // appended fields as their defaults
    a = base_args(h, W, y, m, A);
    a.struct_size = (uint32_t)offsetof(plp_args, global_tokens);
    a.global_tokens = -5;  // ignored: outside the declared size
    size_t n1 = 0;
    CHECK(plp_workspace_size(&a, &n1) == PLP_OK);
  }

  // the other entry points
  {
    size_t bytes = 0;
    CHECK(plp_selective_entropy_workspace_size(0, 256, 1000, PLP_DTYPE_BF16, &bytes) == PLP_E_INVALID);
    CHECK(plp_selective_entropy_workspace_size(100, 256, 1000, 7, &bytes) == PLP_E_INVALID);
    CHECK(plp_selective_entropy_workspace_size(100, 256, 1000, PLP_DTYPE_BF16, nullptr) == PLP_E_INVALID);
    CHECK(plp_selective_entropy_workspace_size(100, 256, 1000, PLP_DTYPE_BF16, &bytes) == PLP_OK && bytes > 0);
    CHECK(plp_selective_entropy(nullptr, W, nullptr, 100, 256, 1000, PLP_DTYPE_BF16, 1.f, nullptr, (float*)out_buf,
                                nullptr, nullptr, 0, nullptr) == PLP_E_INVALID);
    CHECK(plp_selective_entropy(h, W, nullptr, 100, 256, 1000, PLP_DTYPE_BF16, 1.f, nullptr, (float*)out_buf,
                                (float*)out_buf, nullptr, 0, nullptr) == PLP_E_INVALID);  // logp without targets
    CHECK(plp_selective_entropy(h, W, nullptr, 100, 256, 1000, PLP_DTYPE_BF16, -1.f, nullptr, (float*)out_buf,
                                nullptr, nullptr, 0, nullptr) == PLP_E_INVALID);
    CHECK(plp_selective_entropy(h, W, nullptr, 100, 256, 1000, PLP_DTYPE_BF16, 1.f, nullptr, (float*)out_buf,
                                nullptr, nullptr, 0, nullptr) == PLP_E_WORKSPACE);
    size_t prep_bytes = 0;
    CHECK(plp_selective_entropy_prepared_workspace_size(100, 256, 1000, PLP_DTYPE_BF16, &prep_bytes) == PLP_OK &&
          prep_bytes > 0 && prep_bytes < bytes);
    CHECK(plp_selective_entropy_prepared_workspace_size(100, 200, 1000, PLP_DTYPE_BF16, &prep_bytes) ==
          PLP_E_UNSUPPORTED);
    CHECK(plp_selective_entropy_prepared(h, W, nullptr, nullptr, 100, 256, 1000, PLP_DTYPE_BF16, 1.f, nullptr,
                                         (float*)out_buf, nullptr, nullptr, 0, nullptr) == PLP_E_INVALID);
    CHECK(plp_selective_entropy_prepared(h, W, W, nullptr, 100, 256, 1000, PLP_DTYPE_BF16, 1.f, nullptr,
                                         (float*)out_buf, nullptr, nullptr, 0, nullptr) == PLP_E_WORKSPACE);
    CHECK(plp_entropy_quantile_mask_workspace_size(-1, &bytes) == PLP_E_INVALID);
    CHECK(plp_entropy_quantile_mask_workspace_size(100, &bytes) == PLP_OK && bytes > 0);
    CHECK(plp_entropy_quantile_mask((const float*)out_buf, (const uint8_t*)m, 100, 2.0, (uint8_t*)out_buf, nullptr,
                                    nullptr, 0, nullptr) == PLP_E_INVALID);
    CHECK(plp_entropy_quantile_mask(nullptr, (const uint8_t*)m, 100, 0.5, (uint8_t*)out_buf, nullptr, nullptr, 0,
                                    nullptr) == PLP_E_INVALID);
    CHECK(plp_entropy_quantile_mask((const float*)out_buf, (const uint8_t*)m, 100, 0.5, (uint8_t*)out_buf, nullptr,
                                    nullptr, 0, nullptr) == PLP_E_WORKSPACE);
    CHECK(plp_entropy_quantile_mask_noalloc(nullptr, nullptr, -1, 0.5, nullptr, nullptr, nullptr) == PLP_E_INVALID);
    CHECK(plp_entropy_quantile_mask_noalloc(nullptr, nullptr, (int64_t)1 << 31, 0.5, nullptr, nullptr, nullptr) ==
          PLP_E_INVALID);
    CHECK(plp_entropy_quantile_mask_noalloc(nullptr, nullptr, 10, 0.5, nullptr, nullptr, nullptr) == PLP_E_INVALID);
    plp_args a = base_args(nullptr, nullptr, nullptr, m, A);
    a.H = 0;
    a.V = 0;
    CHECK(plp_policy_loss_workspace_size(&a, &bytes) == PLP_OK && bytes > 0);
    CHECK(plp_policy_loss_from_logprobs(&a, nullptr, nullptr, &o, nullptr, 0, nullptr) == PLP_E_INVALID);
    a.top_entropy_quantile = 0.5;
    CHECK(plp_policy_loss_from_logprobs(&a, (const float*)out_buf, nullptr, &o, nullptr, 0, nullptr) ==
          PLP_E_INVALID);  // q < 1 needs entropies
    a.top_entropy_quantile = 1.0;
    CHECK(plp_policy_loss_from_logprobs(&a, (const float*)out_buf, nullptr, &o, nullptr, 0, nullptr) ==
          PLP_E_WORKSPACE);
    CHECK(plp_prepared_weight_size(896, 151936, PLP_DTYPE_BF16, &bytes) == PLP_OK && bytes == (size_t)151936 * 896 * 2);
    CHECK(plp_prepared_weight_size(896, 151936, PLP_DTYPE_F32, &bytes) == PLP_E_UNSUPPORTED);
    CHECK(plp_prepared_weight_size(896, 151936, PLP_DTYPE_BF16, nullptr) == PLP_E_INVALID);
    CHECK(plp_prepare_weight(W, 128, 1000, PLP_DTYPE_BF16, nullptr, 1 << 20, nullptr) == PLP_E_INVALID);
    CHECK(plp_prepare_weight(W, 128, 1000, PLP_DTYPE_BF16, out_buf, 100, nullptr) == PLP_E_INVALID);
    CHECK(plp_prepare_weight(W, 100, 1000, PLP_DTYPE_BF16, out_buf, 1 << 20, nullptr) == PLP_E_UNSUPPORTED);
    CHECK(plp_profile_start(0) == PLP_E_INVALID);
    CHECK(plp_profile_stop(nullptr, nullptr) == PLP_E_INVALID);
  }
  free(h);
  free(W);
  free(y);
  free(m);
  free(A);
  free(out_buf);
  if (!g_fail) printf("host checks passed\n");
  return g_fail;
}
