// Host-side checks of the C ABI under AddressSanitizer.  The library is built
// with the sanitizer on its host code, and every call below returns during argument validation or planning, before any
// HIP call: the pointers are addresses that are never dereferenced.  A
// sanitizer report, or a return code other than the one expected, fails.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "moe_decode.h"

namespace {

int failures = 0;

void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    std::printf("line %d: %s returned %d, expected %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, code) expect((call), (code), #call, __LINE__)

// Far-apart, 256-byte aligned stand-ins for device buffers (never dereferenced).
template <typename T>
T* at(int slot, uintptr_t plus = 0) {
  return reinterpret_cast<T*>((uintptr_t(slot + 1) << 36) + plus);
}

struct Args {
  const void* x = at<void>(0);
  const int32_t* ids = at<int32_t>(1);
  const float* w = at<float>(2);
  const uint8_t* wg = at<uint8_t>(3);
  const uint8_t* sg = at<uint8_t>(4);
  const uint8_t* wu = at<uint8_t>(5);
  const uint8_t* su = at<uint8_t>(6);
  const uint8_t* wd = at<uint8_t>(7);
  const uint8_t* sd = at<uint8_t>(8);
  void* h = at<void>(9);
  void* y = at<void>(10);
};

int gate_up(const Args& a, int B, int H, int I, int E, int k) {
  return moe_decode_gate_up(a.x, a.ids, a.wg, a.sg, a.wu, a.su, a.h, B, H, I, E, k, nullptr);
}
int down(const Args& a, int B, int H, int I, int E, int k) {
  return moe_decode_down(a.h, a.ids, a.w, a.wd, a.sd, a.y, B, H, I, E, k, nullptr);
}

}  // namespace

int main() {
  // every code has a message
  for (int c = -12; c <= 2; ++c) {
    const char* m = moe_decode_strerror(c);
    if (!m || !std::strlen(m)) {
      std::printf("strerror(%d) is empty\n", c);
      ++failures;
    }
  }

  // the built-in table over a grid of shapes: a plan or a shape/argument error, never anything else
  const int Bs[] = {0, 1, 2, 3, 4, 5, 8, 9, 10, 16, 24, 32, 42, 43, 64, 100, 128, 256, 1024, 5000};
  const int Hs[] = {32, 1024, 2048, 3072, 4096, 6144, 8192, 8224};
  const int Is[] = {32, 96, 768, 1536, 2048, 4096};
  const int Es[] = {1, 8, 22, 128, 512, 1024, 2048};
  const int ks[] = {1, 4, 8, 64};
  long plans = 0;
  for (int B : Bs)
    for (int H : Hs)
      for (int I : Is)
        for (int E : Es)
          for (int k : ks) {
            int v = -1, r = -1, g = -1;
            int rc = moe_decode_gate_up_plan(B, H, I, E, k, &v, &r, &g);
            if (rc == MOE_OK) {
              ++plans;
              if (v < 1 || v > 3 || r < 1 || g < 0) {
                std::printf("gate/up plan B=%d H=%d I=%d E=%d k=%d: %d %d %d\n", B, H, I, E, k, v, r, g);
                ++failures;
              }
            } else if (rc != MOE_ERR_SHAPE && rc != MOE_ERR_ARG) {
              std::printf("gate/up plan B=%d H=%d I=%d E=%d k=%d: rc %d\n", B, H, I, E, k, rc);
              ++failures;
            }
            rc = moe_decode_down_plan(B, H, I, E, k, &v, &r, &g);
            if (rc == MOE_OK) {
              ++plans;
              if (v < 1 || v > 3 || r < 1 || g < 0) {
                std::printf("down plan B=%d H=%d I=%d E=%d k=%d: %d %d %d\n", B, H, I, E, k, v, r, g);
                ++failures;
              }
            } else if (rc != MOE_ERR_SHAPE && rc != MOE_ERR_ARG) {
              std::printf("down plan B=%d H=%d I=%d E=%d k=%d: rc %d\n", B, H, I, E, k, rc);
              ++failures;
            }
            size_t ws = 0;
            rc = moe_decode_conventional_workspace(B, H, I, E, k, &ws);
            if (rc != MOE_OK && rc != MOE_ERR_SHAPE) {
              std::printf("workspace B=%d H=%d I=%d E=%d k=%d: rc %d\n", B, H, I, E, k, rc);
              ++failures;
            }
          }
  if (plans == 0) {
    std::printf("no shape planned\n");
    ++failures;
  }
  int v, r, g;
  EXPECT(moe_decode_gate_up_plan(32, 2048, 768, 128, 8, nullptr, &r, &g), MOE_ERR_NULL);
  EXPECT(moe_decode_down_plan(32, 2048, 768, 128, 8, &v, nullptr, &g), MOE_ERR_NULL);
  EXPECT(moe_decode_conventional_workspace(32, 2048, 768, 128, 8, nullptr), MOE_ERR_NULL);

  const Args a;
  const int B = 32, H = 2048, I = 768, E = 128, k = 8;
  // shapes
  EXPECT(gate_up(a, -1, H, I, E, k), MOE_ERR_SHAPE);
  EXPECT(gate_up(a, B, H + 16, I, E, k), MOE_ERR_SHAPE);
  EXPECT(gate_up(a, B, 8192 + 32, I, E, k), MOE_ERR_SHAPE);
  EXPECT(down(a, B, H, I + 16, E, k), MOE_ERR_SHAPE);
  EXPECT(down(a, B, H, I, 4, 8), MOE_ERR_SHAPE);
  EXPECT(down(a, B, H, 4096, E, 8), MOE_ERR_SHAPE);   // k*I beyond 16384
  // an empty batch touches nothing
  EXPECT(gate_up(a, 0, H, I, E, k), MOE_OK);
  EXPECT(down(a, 0, H, I, E, k), MOE_OK);
  // null pointers
  {
    Args n = a;
    n.wu = nullptr;
    EXPECT(gate_up(n, B, H, I, E, k), MOE_ERR_NULL);
    n = a;
    n.w = nullptr;
    EXPECT(down(n, B, H, I, E, k), MOE_ERR_NULL);
  }
  // alignment
  {
    Args m = a;
    m.x = at<void>(0, 8);
    EXPECT(gate_up(m, B, H, I, E, k), MOE_ERR_ALIGN);
    m = a;
    m.ids = at<int32_t>(1, 2);
    EXPECT(down(m, B, H, I, E, k), MOE_ERR_ALIGN);
  }
  // outputs overlapping inputs
  {
    Args o = a;
    o.h = at<void>(3, 4096);   // inside w_gate
    EXPECT(gate_up(o, B, H, I, E, k), MOE_ERR_ALIAS);
    o = a;
    o.y = at<void>(9, 64);     // inside h
    EXPECT(down(o, B, H, I, E, k), MOE_ERR_ALIAS);
  }
  // tuning arguments
  EXPECT(moe_decode_gate_up_ex(a.x, a.ids, a.wg, a.sg, a.wu, a.su, a.h, B, H, I, E, k, 9, 0, nullptr), MOE_ERR_ARG);
  EXPECT(moe_decode_gate_up_ex(a.x, a.ids, a.wg, a.sg, a.wu, a.su, a.h, B, H, I, E, k, 1, 3, nullptr), MOE_ERR_ARG);
  EXPECT(moe_decode_gate_up_ex(a.x, a.ids, a.wg, a.sg, a.wu, a.su, a.h, B, H, I, E, k, -1, 0, nullptr), MOE_ERR_ARG);
  EXPECT(moe_decode_down_ex(a.h, a.ids, a.w, a.wd, a.sd, a.y, B, H, I, E, k, 3, 4, nullptr), MOE_ERR_ARG);
  EXPECT(moe_decode_down_ex(a.h, a.ids, a.w, a.wd, a.sd, a.y, B, H, I, E, k, 0, -2, nullptr), MOE_ERR_ARG);
  // router
  const float* lg = at<float>(11);
  int32_t* ido = at<int32_t>(12);
  float* two = at<float>(13);
  EXPECT(moe_decode_route(lg, ido, two, B, 2048, k, nullptr), MOE_ERR_SHAPE);   // E beyond 1024
  EXPECT(moe_decode_route(lg, ido, two, B, E, 65, nullptr), MOE_ERR_SHAPE);     // k beyond 64
  EXPECT(moe_decode_route(nullptr, ido, two, B, E, k, nullptr), MOE_ERR_NULL);
  EXPECT(moe_decode_route(lg, at<int32_t>(11, 64), two, B, E, k, nullptr), MOE_ERR_ALIAS);
  EXPECT(moe_decode_gate_up_routed(a.x, lg, a.wg, a.sg, a.wu, a.su, at<void>(11, 64), ido, two, B, H, I, E, k,
                                   nullptr),
         MOE_ERR_ALIAS);
  EXPECT(moe_decode_gate_up_routed_ex(a.x, lg, a.wg, a.sg, a.wu, a.su, a.h, ido, two, B, H, I, E, k, 7, 0, nullptr),
         MOE_ERR_ARG);
  // conventional path
  size_t need = 0;
  EXPECT(moe_decode_conventional_workspace(B, H, I, E, k, &need), MOE_OK);
  if (need == 0 || need % 256) {
    std::printf("workspace size %zu\n", need);
    ++failures;
  }
  void* ws = at<void>(14);
  EXPECT(moe_decode_conventional(a.x, a.ids, a.w, a.wg, a.sg, a.wu, a.su, a.wd, a.sd, a.y, ws, need - 256, B, H, I,
                                 E, k, nullptr),
         MOE_ERR_ARG);
  EXPECT(moe_decode_conventional(a.x, a.ids, a.w, a.wg, a.sg, a.wu, a.su, a.wd, a.sd, a.y, at<void>(0, 256), need, B,
                                 H, I, E, k, nullptr),
         MOE_ERR_ALIAS);
  EXPECT(moe_decode_conventional(a.x, a.ids, a.w, a.wg, a.sg, a.wu, a.su, a.wd, a.sd, a.y, at<void>(14, 16), need, B,
                                 H, I, E, k, nullptr),
         MOE_ERR_ALIGN);
  EXPECT(moe_decode_conventional_noalloc(a.x, a.ids, a.w, a.wg, a.sg, a.wu, a.su, a.wd, a.sd, nullptr, B, H, I, E, k,
                                         nullptr),
         MOE_ERR_NULL);
  // a shape whose workspace exceeds the fixed 32 MiB buffer: refused before any device call
  EXPECT(moe_decode_conventional_noalloc(a.x, a.ids, a.w, a.wg, a.sg, a.wu, a.su, a.wd, a.sd, a.y, 128, 8192, 2048, 16,
                                         8, nullptr),
         MOE_ERR_SCRATCH);
  // bandwidth probes
  EXPECT(moe_decode_copy_peak(at<void>(15), at<void>(16), 100, nullptr), MOE_ERR_SHAPE);
  EXPECT(moe_decode_copy_peak(at<void>(15), at<void>(15, 64), 1024, nullptr), MOE_ERR_ALIAS);
  EXPECT(moe_decode_copy_peak(nullptr, at<void>(16), 1024, nullptr), MOE_ERR_NULL);
  EXPECT(moe_decode_read_peak(at<void>(15, 8), 1024, at<void>(16), nullptr), MOE_ERR_ALIGN);

  std::printf("%ld plans, %d failures\n", plans, failures);
  return failures == 0 ? 0 : 1;
}
