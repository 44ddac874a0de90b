// Host-only exercise of the C ABI (create / get_info / run / run_strided /
// destroy / strerror / adaln_residual) built with AddressSanitizer and
// UndefinedBehaviorSanitizer, against stub kernel launchers that record which
// kernel a plan chose and never touch memory. No GPU is needed: every
// argument check, the plan arithmetic and the span / overlap tests run on the
// host, over a grid of valid and invalid descriptors. Exits nonzero on the
// first broken invariant; the sanitizers abort on any memory or UB error.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "plan.h"
#include "swin3d_wattn.h"

static int g_kernel = 0;
static int g_calls = 0;
#define STUB(name, id)                                                                                  \
  int name(const swin3d_wattn_plan* p, const void*, const void*, const void*, void*,                    \
           const swin3d_wattn_strides_t* st, void*) {                                                   \
    g_kernel = id;                                                                                      \
    ++g_calls;                                                                                          \
    if (p->kernel != id || st->q < (int64_t)p->desc.heads * p->desc.head_dim) std::abort();             \
    return 0;                                                                                           \
  }
STUB(wattn_launch_bf16, 1)
STUB(wattn_launch_f32x3, 2)
STUB(wattn_launch_stream, 3)
STUB(wattn_launch_f32m, 4)
STUB(wattn_launch_window, 5)
int adaln_launch(const swin3d_adaln_desc_t*, const void*, const void*, const float*, const float*, void*, void*) {
  ++g_calls;
  return 0;
}

#define CHECK(c)                                                                  \
  do {                                                                            \
    if (!(c)) {                                                                   \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);        \
      std::exit(1);                                                               \
    }                                                                             \
  } while (0)

static uintptr_t fake(uint64_t byte_offset) { return (uintptr_t)0x100000000ull + (uintptr_t)byte_offset; }

int main() {
  const int32_t dtypes[] = {SWIN3D_WATTN_BF16, SWIN3D_WATTN_F32, SWIN3D_WATTN_F32_SPLIT, 7, -1};
  const int32_t hds[] = {0, 32, 64, 96, 128, 256};
  const int32_t wins[][3] = {{2, 6, 12}, {2, 12, 12}, {1, 1, 1}, {16, 16, 16}, {17, 16, 16}, {0, 6, 12},
                             {4, 12, 24}, {3, 12, 12}, {1, 7, 7}, {2, 6, 6}};
  const int32_t shifts[][3] = {{0, 0, 0}, {1, 3, 6}, {-1, 0, 0}, {1, 6, 6}, {2, 6, 12}};
  const int32_t grids[][4] = {{1, 4, 180, 360}, {2, 3, 10, 14}, {1, 1, 1, 1}, {0, 4, 4, 4}, {1, 5, 13, 17},
                              {1, 1 << 24, 1, 1}, {3, 2, 12, 24}};
  const int32_t headss[] = {1, 8, 65535, 65536, 0};
  const float scales[] = {0.125f, NAN};
  const float biases[] = {-100.0f, -INFINITY, 1.0f};
  long made = 0, refused = 0;
  for (int32_t dt : dtypes)
    for (int32_t hd : hds)
      for (auto& w : wins)
        for (auto& s : shifts)
          for (auto& g : grids)
            for (int32_t heads : headss)
              for (float sc : scales)
                for (float bias : biases) {
                  swin3d_wattn_desc_t d;
                  std::memset(&d, 0, sizeof d);
                  d.B = g[0], d.D = g[1], d.H = g[2], d.W = g[3];
                  d.heads = heads, d.head_dim = hd;
                  for (int a = 0; a < 3; ++a) d.window[a] = w[a], d.shift[a] = s[a];
                  d.dtype = dt, d.scale = sc, d.cross_region_bias = bias;
                  swin3d_wattn_t plan = (swin3d_wattn_t)0x1;
                  const int rc = swin3d_wattn_create(&d, &plan);
                  if (rc != 0) {
                    CHECK(rc == SWIN3D_WATTN_EINVAL || rc == SWIN3D_WATTN_EUNSUPPORTED);
                    CHECK(plan == nullptr);
                    ++refused;
                    continue;
                  }
                  ++made;
                  swin3d_wattn_info_t info;
                  CHECK(swin3d_wattn_get_info(plan, &info) == 0);
                  CHECK(info.kernel >= 1 && info.kernel <= 5);
                  CHECK(info.workgroups > 0 && info.threads_per_workgroup > 0);
                  CHECK(info.n_windows > 0 && info.n_masked_windows >= 0 && info.n_masked_windows <= info.n_windows);
                  CHECK(info.tokens == (int64_t)d.B * d.D * d.H * d.W);
                  CHECK(info.tokens_per_window == w[0] * w[1] * w[2]);
                  const int32_t X[3] = {d.D, d.H, d.W};
                  for (int a = 0; a < 3; ++a)
                    CHECK(info.padded[a] == info.windows_per_axis[a] * w[a] && info.padded[a] >= X[a]);
                  const int64_t row = (int64_t)heads * hd;
                  const int64_t esz = dt == SWIN3D_WATTN_BF16 ? 2 : 4;
                  const uint64_t bytes = (uint64_t)info.tokens * row * esz;
                  // contiguous run on disjoint spans, then a fused-QKV view with O beside it
                  const uintptr_t q = fake(0), k = fake(bytes), v = fake(2 * bytes), o = fake(3 * bytes + 4096);
                  g_kernel = 0;
                  CHECK(swin3d_wattn_run(plan, (void*)q, (void*)k, (void*)v, (void*)o, nullptr) == 0);
                  CHECK(g_kernel == info.kernel);
                  swin3d_wattn_strides_t st{3 * row, 3 * row, 3 * row, row};
                  const int rs = swin3d_wattn_run_strided(plan, (void*)q, (void*)(q + row * esz), (void*)(q + 2 * row * esz),
                                                          (void*)fake(3 * bytes + 8192), &st, nullptr);
                  CHECK(rs == 0 || rs == SWIN3D_WATTN_EINVAL);  // EINVAL only where 3 * row breaks a stride limit
                  // refused: O overlapping Q, misaligned pointers, null pointers, strides too small
                  CHECK(swin3d_wattn_run(plan, (void*)q, (void*)k, (void*)v, (void*)(q + 16), nullptr) == SWIN3D_WATTN_EINVAL);
                  CHECK(swin3d_wattn_run(plan, (void*)(q + 2), (void*)k, (void*)v, (void*)o, nullptr) == SWIN3D_WATTN_EINVAL);
                  CHECK(swin3d_wattn_run(plan, nullptr, (void*)k, (void*)v, (void*)o, nullptr) == SWIN3D_WATTN_EINVAL);
                  swin3d_wattn_strides_t bad{row - 1, row, row, row};
                  CHECK(swin3d_wattn_run_strided(plan, (void*)q, (void*)k, (void*)v, (void*)o, &bad, nullptr) ==
                        SWIN3D_WATTN_EINVAL);
                  CHECK(swin3d_wattn_run_strided(plan, (void*)q, (void*)k, (void*)v, (void*)o, nullptr, nullptr) ==
                        SWIN3D_WATTN_EINVAL);
                  CHECK(swin3d_wattn_destroy(plan) == 0);
                }
  CHECK(swin3d_wattn_destroy(nullptr) == 0);
  CHECK(swin3d_wattn_create(nullptr, nullptr) == SWIN3D_WATTN_EINVAL);
  swin3d_wattn_info_t info;
  CHECK(swin3d_wattn_get_info(nullptr, &info) == SWIN3D_WATTN_EINVAL);
  for (int code = -10; code <= 10; ++code) CHECK(swin3d_wattn_strerror(code) != nullptr);
  CHECK(swin3d_wattn_run(nullptr, (void*)fake(0), (void*)fake(64), (void*)fake(128), (void*)fake(256), nullptr) ==
        SWIN3D_WATTN_EINVAL);

  // AdaLN descriptors
  long adaln_ok = 0;
  const int64_t rowss[] = {1, 700, 259200, 0, -3};
  const int32_t Bs[] = {1, 2, 0};
  const int32_t Cs[] = {256, 512, 1000, 4096, 4352, 0};
  const int32_t adt[] = {SWIN3D_WATTN_F32, SWIN3D_WATTN_BF16, 5};
  const float epss[] = {1e-5f, 0.0f, NAN, INFINITY};
  for (int64_t rows : rowss)
    for (int32_t B : Bs)
      for (int32_t C : Cs)
        for (int32_t xd : adt)
          for (int32_t rd : adt)
            for (int32_t od : adt)
              for (float eps : epss) {
                swin3d_adaln_desc_t a{rows, B, C, xd, rd, od, eps};
                const uint64_t n = (rows > 0 && B > 0 && C > 0) ? (uint64_t)rows * B * C * 4 : 64;
                const uintptr_t x = fake(0), res = fake(n + 256), gb = fake(2 * n + 512), out = fake(3 * n + 1024);
                const int rc = swin3d_adaln_residual(&a, (void*)x, (void*)res, (const float*)gb,
                                                     (const float*)(gb + 16 * 4096), (void*)out, nullptr);
                CHECK(rc == 0 || rc == SWIN3D_WATTN_EINVAL || rc == SWIN3D_WATTN_EUNSUPPORTED);
                adaln_ok += rc == 0;
                CHECK(swin3d_adaln_residual(&a, nullptr, (void*)res, (const float*)gb, (const float*)gb,
                                            (void*)out, nullptr) != 0);
              }
  CHECK(swin3d_adaln_residual(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == SWIN3D_WATTN_EINVAL);
  CHECK(made > 100 && refused > 100 && adaln_ok > 10);
  std::printf("ok: %ld plans made, %ld refused, %ld adaln launches, %d stub launches\n", made, refused, adaln_ok,
              g_calls);
  return 0;
}
