// Host-side checks of libk2's C ABI built with AddressSanitizer and UndefinedBehaviorSanitizer on the
// host code: every call below fails validation (or only queries sizes / layouts) before any device
// work, so it runs without a GPU. Fake device addresses are never dereferenced. Exit status 0 when
// every status matches; the sanitizers abort on an invalid access or undefined behaviour.
#include <cstdint>
#include <cstdio>

#include "k2.h"

static int failures = 0;
#define EXPECT(call, want)                                                                        \
  do {                                                                                            \
    const long got_ = (long)(call);                                                               \
    if (got_ != (long)(want)) {                                                                   \
      std::printf("FAIL %s:%d: %s = %ld, expected %ld (%s)\n", __FILE__, __LINE__, #call, got_,   \
                  (long)(want), k2_last_error());                                                 \
      ++failures;                                                                                 \
    }                                                                                             \
  } while (0)

int main() {
  const uintptr_t F = 0x7F0000000000ull;  // fake, 256-byte aligned device address
  auto fp = [&](int i) { return (void*)(F + 0x1000000ull * (uintptr_t)i); };
  k2_block_cfg c;
  k2_block_cfg_default(&c);
  k2_block_weights w = {};
  w.scale_shift_table = (const float*)fp(1);
  w.norm1_w = (const float*)fp(2); w.norm2_w = (const float*)fp(3);
  w.norm_q_w = (const float*)fp(4); w.norm_k_w = (const float*)fp(5);
  w.to_q = fp(6); w.to_k = fp(7); w.to_v = fp(8); w.to_gate = fp(9);
  w.to_out = fp(10); w.ff_gate = fp(11); w.ff_up = fp(12); w.ff_down = fp(13);
  const float* h = (const float*)fp(20);
  float* o = (float*)fp(21);
  const float* temb = (const float*)fp(22);
  const float* pos = (const float*)fp(23);

  // sizes and layouts over a range of shapes (the workspace carving)
  const int shapes[][3] = {{1, 0, 1}, {1, 4, 4}, {2, 512, 4096}, {1, 512, 16384}, {1024, 0, 12}, {3, 7, 33}};
  for (const auto& s : shapes) {
    const size_t need = k2_block_workspace_bytes(&c, s[0], s[1], s[2]);
    k2_block_workspace_layout lay;
    EXPECT(k2_block_workspace_layout_query(&c, s[0], s[1], s[2], &lay), K2_OK);
    if (lay.total != need || lay.a < lay.x2 || lay.x2 < lay.og || lay.ldvt < s[1] + s[2]) {
      std::printf("FAIL layout for (%d, %d, %d)\n", s[0], s[1], s[2]);
      ++failures;
    }
    if (k2_block_backward_workspace_bytes(&c, s[0], s[1], s[2]) < need / 2) {
      std::printf("FAIL backward workspace for (%d, %d, %d)\n", s[0], s[1], s[2]);
      ++failures;
    }
  }
  // validation failures, each before any launch
  EXPECT(k2_block_forward(nullptr, &w, 1, 4, 4, h, o, temb, pos, 8, 3, nullptr, fp(30), 0, nullptr), K2_ERR_NULL);
  EXPECT(k2_block_forward(&c, &w, 1, 4, 4, h, o, temb, pos, 7, 3, nullptr, fp(30), 0, nullptr), K2_ERR_SHAPE);
  EXPECT(k2_block_forward(&c, &w, 0, 4, 4, h, o, temb, pos, 8, 3, nullptr, fp(30), 0, nullptr), K2_ERR_SHAPE);
  EXPECT(k2_block_forward(&c, &w, 1, 4, 4, h, o, temb, pos, 8, 3, nullptr, fp(30), 0, nullptr), K2_ERR_WORKSPACE);
  EXPECT(k2_block_forward(&c, &w, 1, 4, 4, (const float*)((char*)h + 4), o, temb, pos, 8, 3, nullptr, fp(30),
                          1 << 30, nullptr), K2_ERR_ALIGN);
  EXPECT(k2_block_forward(&c, &w, 2, 512, 1400000, h, o, temb, pos, 1400512, 3, nullptr, fp(30), 0, nullptr),
         K2_ERR_SHAPE);
  EXPECT(k2_block_forward(&c, &w, 65535, 512, 40000, h, o, temb, pos, 40512, 3, nullptr, fp(30), 0, nullptr),
         K2_ERR_SHAPE);
  k2_block_cfg bad = c;
  bad.axes_dims[0] = 30;
  EXPECT(k2_block_forward(&bad, &w, 1, 4, 4, h, o, temb, pos, 8, 3, nullptr, fp(30), 0, nullptr), K2_ERR_CONFIG);
  bad = c;
  bad.num_kv_heads = 16;
  EXPECT(k2_block_forward(&bad, &w, 1, 4, 4, h, o, temb, pos, 8, 3, nullptr, fp(30), 0, nullptr), K2_ERR_CONFIG);
  bad = c;
  bad.dtype = (k2_dtype)7;
  EXPECT(k2_block_forward(&bad, &w, 1, 4, 4, h, o, temb, pos, 8, 3, nullptr, fp(30), 0, nullptr), K2_ERR_DTYPE);
  EXPECT(k2_block_forward_static_ws(&c, &w, 2, 512, 4096, h, o, temb, pos, 4608, 3, nullptr, nullptr),
         K2_ERR_WORKSPACE);
  k2_block_grads gr = {};
  EXPECT(k2_block_backward(&c, &w, 1, 4, 4, h, temb, pos, 8, 3, nullptr, nullptr, o, nullptr, &gr, fp(30), 0, nullptr),
         K2_ERR_NULL);
  EXPECT(k2_mfma_rate_probe(0, 1, o, nullptr), K2_ERR_SHAPE);
  EXPECT(k2_cfg_euler_update(nullptr, o, h, nullptr, 16, 0.0f, 1.0f, 0.5f, nullptr), K2_ERR_NULL);
  // the sampler's host-side sigma grid
  float sig[29];
  EXPECT(k2_flow_sigmas(nullptr, 28, 4096, 0, sig), K2_OK);
  if (!(sig[0] > 0.99f && sig[28] == 0.0f)) {
    std::printf("FAIL sigma grid ends\n");
    ++failures;
  }
  std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "OK", failures);
  return failures ? 1 : 0;
}
