// Host-side argument checks of the C-ABI, run under AddressSanitizer with no GPU present.
//
// Every call below must return its status before anything touches the device: descriptor
// and size checks, null and alignment checks, workspace sizing, the scratch limit of the
// allocation-free entry point, the chain's per-layer checks, and the status strings.  Device
// pointers are stand-ins that the checks look at but never dereference.  The sanitizer
// reports any out-of-bounds or invalid host access these paths make; the exit status counts
// the calls that returned something other than the expected status.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/moe_iq4nl.h"

static int g_fail = 0;

static void expect(const char* what, moe_status got, moe_status want) {
  if (got != want) {
    std::printf("FAIL %s: got %d want %d\n", what, (int)got, (int)want);
    ++g_fail;
  }
}

static moe_desc make(int H, int F, int E, int k, int S, int gating, int renorm, int maxT) {
  moe_desc d;
  std::memset(&d, 0, sizeof d);
  d.hidden = H; d.ffn = F; d.n_experts = E; d.top_k = k; d.n_shared = S;
  d.gating = gating; d.renormalize = renorm; d.max_tokens = maxT;
  return d;
}

int main() {
  alignas(256) static unsigned char fake_dev[1 << 12];      // never dereferenced by the checks
  const float* fx = reinterpret_cast<const float*>(fake_dev);
  float* fy = reinterpret_cast<float*>(fake_dev);
  const moe_desc good = make(3584, 1024, 64, 4, 1, MOE_GATING_SIGMOID, 1, 16);
  const int64_t esz = 3 * (int64_t)1024 * (3584 / 32) * 18;
  moe_bank bank{fake_dev, (esz + 15) / 16 * 16};

  // workspace sizing over shapes and token counts (host arithmetic only)
  const int shapes[][5] = {{3584, 1024, 64, 4, 1}, {2048, 512, 512, 10, 1}, {7168, 1536, 384, 6, 1},
                           {256, 128, 8, 2, 1},    {64, 64, 1, 1, 0},       {8192, 8192, 1023, 32, 1}};
  size_t prev = 0, bytes = 0;
  for (const auto& s : shapes) {
    const moe_desc d = make(s[0], s[1], s[2], s[3], s[4], MOE_GATING_SOFTMAX, 0, 8192);
    // non-decreasing within the fused-decode range (T <= 16) and beyond it (the decode layout
    // is sized for T <= 16 only, so T = 17 may need less than T = 16)
    prev = 0;
    for (int T : {0, 1, 2, 3, 4, 5, 15, 16, -17, 64, 2048, 8192, 100000}) {
      if (T < 0) { T = -T; prev = 0; }
      expect("workspace_size", moe_workspace_size(&d, T, &bytes), MOE_OK);
      if (bytes < 256 || bytes < prev) { std::printf("FAIL workspace %zu after %zu\n", bytes, prev); ++g_fail; }
      prev = bytes;
    }
    expect("workspace_size T<0", moe_workspace_size(&d, -1, &bytes), MOE_ERR_SHAPE);
  }
  expect("workspace_size null bytes", moe_workspace_size(&good, 1, nullptr), MOE_ERR_NULL);
  expect("workspace_size null desc", moe_workspace_size(nullptr, 1, &bytes), MOE_ERR_NULL);

  // descriptors out of range
  struct { const char* what; moe_desc d; moe_status want; } bad[] = {
      {"hidden 100", make(100, 1024, 64, 4, 1, 0, 1, 16), MOE_ERR_SHAPE},
      {"hidden 16384", make(16384, 1024, 64, 4, 1, 0, 1, 16), MOE_ERR_SHAPE},
      {"ffn 32", make(3584, 32, 64, 4, 1, 0, 1, 16), MOE_ERR_SHAPE},
      {"top_k 0", make(3584, 1024, 64, 0, 1, 0, 1, 16), MOE_ERR_SHAPE},
      {"top_k > E", make(3584, 1024, 4, 5, 1, 0, 1, 16), MOE_ERR_SHAPE},
      {"top_k 33", make(3584, 1024, 64, 33, 1, 0, 1, 16), MOE_ERR_SHAPE},
      {"n_shared 2", make(3584, 1024, 64, 4, 2, 0, 1, 16), MOE_ERR_SHAPE},
      {"E + S 1025", make(3584, 1024, 1024, 4, 1, 0, 1, 16), MOE_ERR_SHAPE},
      {"gating 7", make(3584, 1024, 64, 4, 1, 7, 1, 16), MOE_ERR_UNSUPPORTED},
      {"renorm 2", make(3584, 1024, 64, 4, 1, 0, 2, 16), MOE_ERR_UNSUPPORTED},
      {"max_tokens 0", make(3584, 1024, 64, 4, 1, 0, 1, 0), MOE_ERR_SHAPE},
  };
  for (const auto& b : bad) {
    expect(b.what, moe_workspace_size(&b.d, 1, &bytes), b.want);
    expect(b.what, moe_route(&b.d, fx, fx, nullptr, 1, nullptr, nullptr, nullptr, fake_dev,
                             sizeof fake_dev, nullptr), b.want);
    expect(b.what, moe_decode_layer(&b.d, &bank, fx, nullptr, fx, 1, 1e-6f, nullptr, fy,
                                    nullptr, nullptr, MOE_DECODE_ALL, fake_dev, sizeof fake_dev,
                                    nullptr), b.want);
    expect(b.what, moe_decode_layer_noalloc(&b.d, &bank, fx, nullptr, fx, 1, 1e-6f, nullptr, fy,
                                            nullptr, nullptr, MOE_DECODE_ALL, nullptr), b.want);
  }

  // banks, stages, sizes, pointers, alignment, workspace
  moe_bank small{fake_dev, 16};
  moe_bank unaligned{fake_dev + 4, bank.expert_stride};
  expect("bank stride", moe_decode_layer(&good, &small, fx, nullptr, fx, 1, 1e-6f, nullptr, fy,
                                         nullptr, nullptr, MOE_DECODE_ALL, fake_dev,
                                         sizeof fake_dev, nullptr), MOE_ERR_SHAPE);
  expect("bank alignment", moe_decode_layer(&good, &unaligned, fx, nullptr, fx, 1, 1e-6f, nullptr,
                                            fy, nullptr, nullptr, MOE_DECODE_ALL, fake_dev,
                                            sizeof fake_dev, nullptr), MOE_ERR_ALIGNMENT);
  expect("null bank", moe_decode_layer(&good, nullptr, fx, nullptr, fx, 1, 1e-6f, nullptr, fy,
                                       nullptr, nullptr, MOE_DECODE_ALL, fake_dev,
                                       sizeof fake_dev, nullptr), MOE_ERR_NULL);
  for (int st : {0, 8, -1})
    expect("stages", moe_decode_layer(&good, &bank, fx, nullptr, fx, 1, 1e-6f, nullptr, fy,
                                      nullptr, nullptr, st, fake_dev, sizeof fake_dev, nullptr),
           MOE_ERR_UNSUPPORTED);
  expect("decode T 17", moe_decode_layer(&good, &bank, fx, nullptr, fx, 17, 1e-6f, nullptr, fy,
                                         nullptr, nullptr, MOE_DECODE_ALL, fake_dev,
                                         sizeof fake_dev, nullptr), MOE_ERR_SHAPE);
  expect("decode null x", moe_decode_layer(&good, &bank, fx, nullptr, nullptr, 1, 1e-6f, nullptr,
                                           fy, nullptr, nullptr, MOE_DECODE_ALL, fake_dev,
                                           sizeof fake_dev, nullptr), MOE_ERR_NULL);
  expect("decode unaligned y",
         moe_decode_layer(&good, &bank, fx, nullptr, fx, 1, 1e-6f, nullptr, fy + 1, nullptr,
                          nullptr, MOE_DECODE_ALL, fake_dev, sizeof fake_dev, nullptr),
         MOE_ERR_ALIGNMENT);
  expect("decode NaN eps", moe_decode_layer(&good, &bank, fx, nullptr, fx, 1, 0.0f / 0.0f, nullptr,
                                            fy, nullptr, nullptr, MOE_DECODE_ALL, fake_dev,
                                            sizeof fake_dev, nullptr), MOE_ERR_SHAPE);
  expect("decode null ws", moe_decode_layer(&good, &bank, fx, nullptr, fx, 1, 1e-6f, nullptr, fy,
                                            nullptr, nullptr, MOE_DECODE_ALL, nullptr, 0, nullptr),
         MOE_ERR_NULL);
  expect("decode small ws", moe_decode_layer(&good, &bank, fx, nullptr, fx, 16, 1e-6f, nullptr,
                                             fy, nullptr, nullptr, MOE_DECODE_ALL, fake_dev, 256,
                                             nullptr), MOE_ERR_WORKSPACE);
  expect("decode T 0", moe_decode_layer(&good, &bank, nullptr, nullptr, nullptr, 0, 1e-6f, nullptr,
                                        nullptr, nullptr, nullptr, MOE_DECODE_ALL, nullptr, 0,
                                        nullptr), MOE_OK);

  // the allocation-free entry point refuses what its fixed scratch cannot hold
  const moe_desc huge = make(8192, 8192, 1023, 32, 1, MOE_GATING_SOFTMAX, 1, 16);
  const int64_t hsz = 3 * (int64_t)8192 * (8192 / 32) * 18;
  moe_bank hbank{fake_dev, (hsz + 15) / 16 * 16};
  expect("noalloc limit", moe_decode_layer_noalloc(&huge, &hbank, fx, nullptr, fx, 16, 1e-6f,
                                                   nullptr, fy, nullptr, nullptr, MOE_DECODE_ALL,
                                                   nullptr), MOE_ERR_SCRATCH_LIMIT);

  // the chain checks every layer before launching anything
  std::vector<moe_layer> layers(3, moe_layer{bank, fx, nullptr});
  layers[2].w_router = nullptr;
  expect("chain null router", moe_decode_chain(&good, layers.data(), 3, fy, 1, 1e-6f, nullptr,
                                               nullptr, fake_dev, sizeof fake_dev, nullptr),
         MOE_ERR_NULL);
  layers[2] = moe_layer{small, fx, nullptr};
  expect("chain bad bank", moe_decode_chain(&good, layers.data(), 3, fy, 1, 1e-6f, nullptr,
                                            nullptr, fake_dev, sizeof fake_dev, nullptr),
         MOE_ERR_SHAPE);
  expect("chain too many", moe_decode_chain(&good, layers.data(), MOE_CHAIN_MAX_LAYERS + 1, fy, 1,
                                            1e-6f, nullptr, nullptr, fake_dev, sizeof fake_dev,
                                            nullptr), MOE_ERR_SHAPE);
  expect("chain null layers", moe_decode_chain(&good, nullptr, 2, fy, 1, 1e-6f, nullptr, nullptr,
                                               fake_dev, sizeof fake_dev, nullptr), MOE_ERR_NULL);
  layers[2] = moe_layer{bank, fx, nullptr};
  int32_t ids[4];
  expect("chain ids without w", moe_decode_chain(&good, layers.data(), 3, fy, 1, 1e-6f, ids,
                                                 nullptr, fake_dev, sizeof fake_dev, nullptr),
         MOE_ERR_NULL);
  expect("chain small ws", moe_decode_chain(&good, layers.data(), 3, fy, 16, 1e-6f, nullptr,
                                            nullptr, fake_dev, 256, nullptr), MOE_ERR_WORKSPACE);

  // other entry points: sizes and pointers
  expect("gemv stage 2", moe_expert_gemv_iq4nl(&good, 2, &bank, nullptr, nullptr, fx, fy, 1,
                                               fake_dev, sizeof fake_dev, nullptr),
         MOE_ERR_UNSUPPORTED);
  expect("gemm stage 5", moe_grouped_gemm_iq4nl(&good, 5, &bank, nullptr, fx, fy, 1, fake_dev,
                                                sizeof fake_dev, nullptr), MOE_ERR_UNSUPPORTED);
  expect("combine T<0", moe_combine(&good, fx, nullptr, fx, -1, nullptr, fy, nullptr),
         MOE_ERR_SHAPE);
  expect("rmsnorm hidden 3", moe_rmsnorm(fx, 1, 3, 1e-6f, fy, nullptr), MOE_ERR_SHAPE);
  expect("rmsnorm eps<0", moe_rmsnorm(fx, 1, 64, -1.0f, fy, nullptr), MOE_ERR_SHAPE);
  expect("rmsnorm null", moe_rmsnorm(nullptr, 1, 64, 1e-6f, fy, nullptr), MOE_ERR_NULL);
  expect("quantize n<0", moe_quantize_iq4nl(fx, -1, fake_dev, nullptr), MOE_ERR_SHAPE);
  expect("dequantize n<0", moe_dequantize_iq4nl(fake_dev, -1, fy, nullptr), MOE_ERR_SHAPE);

  for (int s = -3; s < 12; ++s) {
    const char* str = moe_status_string(s);
    if (!str || !str[0]) { std::printf("FAIL status string %d\n", s); ++g_fail; }
  }
  if (moe_abi_version() != MOE_ABI_VERSION) { std::printf("FAIL abi version\n"); ++g_fail; }
  std::printf("%d failures\n", g_fail);
  return g_fail != 0;
}
