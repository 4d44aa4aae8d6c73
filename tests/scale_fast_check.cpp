// Host check of the device codec's branch-free E4M3 block scale
// (e4m3_scale_fast) against the oracle's brute-force nearest-code search
// (release post of the gzenz/ninfer fork, "NVFP4 KV cache (from scratch)",
// bullet 1: E4M3 block scales).  Samples: every binary32 within 256 ulps of
// 6 * v and of 6 * (v + v') / 2 for every pair of neighbouring E4M3 values
// (the places where the choice changes or ties), the saturation edges,
// zero, subnormals, +infinity, and 2^20 random bit patterns below 2^13.
// Prints the number of mismatches and the first few; exits 1 on any.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "nvfp4kv_codec.hpp"

extern "C" int orc_e4m3_scale_code(float amax);
extern "C" double orc_e4m3_value(int code);

static float f_of(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }

int main() {
  std::vector<float> xs;
  auto around = [&](float c, int n) {
    const uint32_t u = u_of(c);
    for (int k = -n; k <= n; ++k) {
      const int64_t v = (int64_t)u + k;
      if (v >= 0 && v <= 0x7F800000) xs.push_back(f_of((uint32_t)v));
    }
  };
  for (int c = 0; c < 127; ++c) {
    const double v = orc_e4m3_value(c);
    around((float)(6.0 * v), 256);
    if (c < 126) around((float)(3.0 * (v + orc_e4m3_value(c + 1))), 256);
  }
  for (float c : {0.0f, 6.0f * 448.0f, 6.0f * 464.0f, 6.0f * 480.0f, 6.0f * 0x1p-10f, 6.0f * 0x1p-6f})
    around(c, 4096);
  for (uint32_t u = 0; u < 65536; ++u) xs.push_back(f_of(u));   // subnormals from zero up
  xs.push_back(f_of(0x7F7FFFFFu));
  xs.push_back(INFINITY);
  std::mt19937 rng(7);
  for (int i = 0; i < (1 << 20); ++i) xs.push_back(f_of(rng() % u_of(8192.0f)));
  long bad = 0;
  for (float a : xs) {
    uint32_t code;
    const float s = nvfp4kv::e4m3_scale_fast(a, code);
    const int want = orc_e4m3_scale_code(a);
    if ((int)code != want || (double)s != orc_e4m3_value(want)) {
      if (bad < 8) std::printf("amax %a: fast %u %a, oracle %d %a\n", a, code, s, want, orc_e4m3_value(want));
      ++bad;
    }
  }
  std::printf("%zu samples, %ld mismatches\n", xs.size(), bad);
  return bad ? 1 : 0;
}
