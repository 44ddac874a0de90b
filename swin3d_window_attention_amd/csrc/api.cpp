// Host side of the C ABI: argument checks and plan geometry. Nothing here
// touches a device, so plans can be built and validated without a GPU.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>

#include "plan.h"

namespace {

constexpr double kLog2e = 1.4426950408889634073599246810019;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Per-axis flags of each window index along one axis: `cut` when the window
// holds two shift regions (the last window along a shifted axis), `pad` when
// one of its positions maps to padding. Shifted position p holds grid
// position (p + s) mod P, so the padding lands at p in [X - s, P - s), which
// need not be the last window; hence the scan.
void axis_flags(int32_t X, int32_t w, int32_t s, int32_t P, int32_t n, bool* cut, bool* pad) {
  for (int32_t kw = 0; kw < n; ++kw) {
    cut[kw] = (s > 0) && (kw == n - 1);
    bool any_pad = false;
    for (int32_t o = 0; o < w; ++o) {
      int32_t p = kw * w + o;
      int32_t g = p + s;
      if (g >= P) g -= P;
      if (g >= X) any_pad = true;
    }
    pad[kw] = any_pad;
  }
}

bool bad_dim(int32_t v) { return v <= 0; }

uint16_t bf16_rne(double x) {
  float f = (float)x;
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

}  // namespace

extern "C" int swin3d_wattn_create(const swin3d_wattn_desc_t* desc, swin3d_wattn_t* out) {
  if (out) *out = nullptr;
  if (!desc || !out) return SWIN3D_WATTN_EINVAL;
  const swin3d_wattn_desc_t& d = *desc;
  if (bad_dim(d.B) || bad_dim(d.D) || bad_dim(d.H) || bad_dim(d.W) || bad_dim(d.heads) ||
      bad_dim(d.head_dim))
    return SWIN3D_WATTN_EINVAL;
  for (int a = 0; a < 3; ++a) {
    if (d.window[a] <= 0) return SWIN3D_WATTN_EINVAL;
    if (d.shift[a] < 0 || d.shift[a] >= d.window[a]) return SWIN3D_WATTN_EINVAL;
  }
  if (d.dtype != SWIN3D_WATTN_F32 && d.dtype != SWIN3D_WATTN_BF16 && d.dtype != SWIN3D_WATTN_F32_SPLIT)
    return SWIN3D_WATTN_EINVAL;
  if (!std::isfinite(d.scale) || !(d.scale > 0.0f)) return SWIN3D_WATTN_EINVAL;
  if (std::isnan(d.cross_region_bias) || d.cross_region_bias > 0.0f) return SWIN3D_WATTN_EINVAL;

  const int32_t X[3] = {d.D, d.H, d.W};
  // the kernels' per-lane index arithmetic takes grid extents below 2^24
  for (int a = 0; a < 3; ++a)
    if (X[a] >= (1 << 24)) return SWIN3D_WATTN_EUNSUPPORTED;
  int64_t tokens = (int64_t)d.B * d.D * d.H * d.W;
  if (tokens >= (int64_t(1) << 31)) return SWIN3D_WATTN_EUNSUPPORTED;
  int64_t padded_tokens = d.B;
  int32_t P[3], nwin[3];
  for (int a = 0; a < 3; ++a) {
    int64_t pa = ceil_div(X[a], d.window[a]) * d.window[a];
    if (pa >= (int64_t(1) << 30)) return SWIN3D_WATTN_EUNSUPPORTED;
    P[a] = (int32_t)pa;
    nwin[a] = (int32_t)(pa / d.window[a]);
    padded_tokens *= pa;
  }
  if (padded_tokens >= (int64_t(1) << 31)) return SWIN3D_WATTN_EUNSUPPORTED;
  const int64_t N64 = (int64_t)d.window[0] * d.window[1] * d.window[2];
  if (N64 > 4096) return SWIN3D_WATTN_EUNSUPPORTED;
  const int32_t N = (int32_t)N64;

  int32_t kernel = -1, threads = 0;
  if (d.dtype == SWIN3D_WATTN_BF16 || d.dtype == SWIN3D_WATTN_F32_SPLIT) {
    // the launch grid is (window [x query block], head); its second dimension stays below 2^16
    if (d.head_dim == 64 && N == 144 && d.heads < 65536) {
      kernel = d.dtype == SWIN3D_WATTN_BF16 ? 1 : 2;
      threads = 256;
    } else if (d.dtype == SWIN3D_WATTN_BF16 && ((d.head_dim == 128 && N == 144) || (d.head_dim == 64 && N == 288)) &&
               d.heads < 65536) {
      kernel = 5;  // the whole window's K and V in LDS, two workgroups per CU
      threads = 256;
    } else if (d.dtype == SWIN3D_WATTN_BF16 && (d.head_dim == 32 || d.head_dim == 64 || d.head_dim == 128) &&
               d.heads < 65536) {
      kernel = 3;  // K and V streamed through LDS
      // block shape: 3 waves / 48-key chunks where that wastes no slot and 64 would, else 4 / 64
      threads = (N % 64 != 0 && N % 48 == 0) ? 192 : 256;
    }
  } else {
    if ((d.head_dim == 32 || d.head_dim == 64) && N <= 256 && d.heads < 65536) {
      kernel = 4;  // FP32 on the matrix cores (tiles of 16 slots, the last one padded)
      threads = 256;
    }
  }
  if (kernel < 0) return SWIN3D_WATTN_EUNSUPPORTED;

  int64_t elems = tokens * d.heads * d.head_dim;
  int64_t n_windows = (int64_t)d.B * nwin[0] * nwin[1] * nwin[2];
  // launch grid (gx, heads): gx = windows, or for kernel 3 windows padded to a
  // multiple of 8 (one XCD per window) x query blocks of 16 slots per wave and
  // query tile, two tiles per wave
  int64_t gx = n_windows;
  if (kernel == 3) {
    const int64_t qblock = (int64_t)(threads / 64) * 16 * 2;
    gx = ceil_div(n_windows, 8) * 8 * ceil_div(N, qblock);
  }
  // a dispatch counts its work-items per grid dimension in 32 bits: gx x threads
  // must stay below 2^32 (reached only by windows of a few tokens on very large grids)
  if (gx * threads >= (int64_t(1) << 32)) return SWIN3D_WATTN_EUNSUPPORTED;
  const int64_t workgroups = gx * d.heads;
  if (workgroups >= (int64_t(1) << 31)) return SWIN3D_WATTN_EUNSUPPORTED;

  // masked-window count (windows needing the region / padding path)
  int64_t masked = 0;
  int32_t special[3][3], padwin[3][2];
  bool bad_special = false;
  {
    bool* flags[3][2];
    for (int a = 0; a < 3; ++a) {
      flags[a][0] = new (std::nothrow) bool[nwin[a]];
      flags[a][1] = new (std::nothrow) bool[nwin[a]];
      if (!flags[a][0] || !flags[a][1]) {
        for (int b = 0; b <= a; ++b) { delete[] flags[b][0]; delete[] flags[b][1]; }
        return SWIN3D_WATTN_EINVAL;
      }
      axis_flags(X[a], d.window[a], d.shift[a], P[a], nwin[a], flags[a][0], flags[a][1]);
    }
    // a window needs the mask path if any axis is cut or padded
    int64_t plain[3];
    for (int a = 0; a < 3; ++a) {
      plain[a] = 0;
      int ns = 0, np = 0;
      for (int j = 0; j < 3; ++j) special[a][j] = -1;
      for (int j = 0; j < 2; ++j) padwin[a][j] = -1;
      for (int32_t i = 0; i < nwin[a]; ++i) {
        if (!flags[a][0][i] && !flags[a][1][i]) {
          ++plain[a];
        } else if (ns < 3) {
          special[a][ns++] = i;
        } else {
          bad_special = true;  // cannot happen: padding spans < one window, plus the last window
        }
        if (flags[a][1][i]) {
          if (np < 2)
            padwin[a][np++] = i;
          else
            bad_special = true;  // cannot happen: padding spans fewer positions than a window
        }
      }
    }
    masked = n_windows - (int64_t)d.B * plain[0] * plain[1] * plain[2];
    for (int a = 0; a < 3; ++a) { delete[] flags[a][0]; delete[] flags[a][1]; }
  }

  if (bad_special) return SWIN3D_WATTN_EUNSUPPORTED;

  swin3d_wattn_plan* p = new (std::nothrow) swin3d_wattn_plan;
  if (!p) return SWIN3D_WATTN_EINVAL;
  std::memset(p, 0, sizeof(*p));
  p->desc = d;
  for (int a = 0; a < 3; ++a) { p->padded[a] = P[a]; p->nwin[a] = nwin[a]; }
  p->n_windows = n_windows;
  p->n_masked_windows = masked;
  p->N = N;
  p->tokens = tokens;
  p->elems = elems;
  p->elem_bytes = d.dtype == SWIN3D_WATTN_BF16 ? 2 : 4;
  p->kernel = kernel;
  p->workgroups = workgroups;
  p->threads = threads;
  p->c2 = (float)((double)d.scale * kLog2e);
  p->bias2 = std::isinf(d.cross_region_bias) ? -INFINITY
                                             : (float)((double)d.cross_region_bias * kLog2e);
  // bias / scale as three bf16 terms (exact to ~2^-24 relative); anything at or
  // beyond -2^100 excludes, like -inf: its exponential is exactly zero
  const double big = -0x1p100;
  double bp = std::isinf(d.cross_region_bias) ? big : (double)d.cross_region_bias / (double)d.scale;
  if (bp < big) bp = big;
  double rest = bp;
  for (int t = 0; t < 3; ++t) {
    p->beta_bf16[t] = bf16_rne(rest);
    rest -= bf16_value(p->beta_bf16[t]);
  }
  p->pad_bf16 = bf16_rne(big);
  for (int a = 0; a < 3; ++a) {
    for (int j = 0; j < 3; ++j) p->special[a][j] = special[a][j];
    for (int j = 0; j < 2; ++j) p->padwin[a][j] = padwin[a][j];
  }
  *out = p;
  return SWIN3D_WATTN_OK;
}

extern "C" int swin3d_wattn_destroy(swin3d_wattn_t plan) {
  delete plan;
  return SWIN3D_WATTN_OK;
}

extern "C" const char* swin3d_wattn_strerror(int code) {
  switch (code) {
    case SWIN3D_WATTN_OK: return "success";
    case SWIN3D_WATTN_EINVAL: return "invalid argument";
    case SWIN3D_WATTN_EUNSUPPORTED: return "unsupported head_dim, window, dtype or size";
    case SWIN3D_WATTN_ELAUNCH: return "kernel launch failed";
    default: return "unknown error code";
  }
}

extern "C" int swin3d_wattn_get_info(swin3d_wattn_t plan, swin3d_wattn_info_t* info) {
  if (!plan || !info) return SWIN3D_WATTN_EINVAL;
  for (int a = 0; a < 3; ++a) {
    info->padded[a] = plan->padded[a];
    info->windows_per_axis[a] = plan->nwin[a];
  }
  info->n_windows = plan->n_windows;
  info->n_masked_windows = plan->n_masked_windows;
  info->tokens_per_window = plan->N;
  info->tokens = plan->tokens;
  info->workgroups = plan->workgroups;
  info->threads_per_workgroup = plan->threads;
  info->kernel = plan->kernel;
  return SWIN3D_WATTN_OK;
}

namespace {
// byte ranges [a, a + a_bytes) and [b, b + b_bytes) intersect (128-bit sums: no wrap-around)
bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  const unsigned __int128 x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (unsigned __int128)b_bytes && y < x + (unsigned __int128)a_bytes;
}
bool misaligned(const void* a) { return ((uintptr_t)a & 15u) != 0; }
}  // namespace

extern "C" int swin3d_wattn_run_strided(swin3d_wattn_t plan, const void* q, const void* k, const void* v,
                                        void* o, const swin3d_wattn_strides_t* st, void* stream) {
  if (!plan || !q || !k || !v || !o || !st) return SWIN3D_WATTN_EINVAL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o)) return SWIN3D_WATTN_EINVAL;
  const int64_t row = (int64_t)plan->desc.heads * plan->desc.head_dim;  // elements per token
  const int64_t s[4] = {st->q, st->k, st->v, st->o};
  int64_t span[4];
  for (int i = 0; i < 4; ++i) {
    if (s[i] < row || s[i] >= (int64_t(1) << 31) || (s[i] * plan->elem_bytes) % 16 != 0) return SWIN3D_WATTN_EINVAL;
    const int64_t elems = (plan->tokens - 1) * s[i] + row;  // < 2^62: tokens and stride are < 2^31
    if (elems > (int64_t(1) << 46)) return SWIN3D_WATTN_EINVAL;  // no device holds such a span
    span[i] = elems * plan->elem_bytes;
  }
  if (overlaps(o, span[3], q, span[0]) || overlaps(o, span[3], k, span[1]) || overlaps(o, span[3], v, span[2]))
    return SWIN3D_WATTN_EINVAL;
  int e;
  switch (plan->kernel) {
    case 1: e = wattn_launch_bf16(plan, q, k, v, o, st, stream); break;
    case 2: e = wattn_launch_f32x3(plan, q, k, v, o, st, stream); break;
    case 3: e = wattn_launch_stream(plan, q, k, v, o, st, stream); break;
    case 4: e = wattn_launch_f32m(plan, q, k, v, o, st, stream); break;
    case 5: e = wattn_launch_window(plan, q, k, v, o, st, stream); break;
    default: return SWIN3D_WATTN_EINVAL;  // not a plan of this library
  }
  return e == 0 ? SWIN3D_WATTN_OK : SWIN3D_WATTN_ELAUNCH;
}

extern "C" int swin3d_wattn_run(swin3d_wattn_t plan, const void* q, const void* k, const void* v,
                                void* o, void* stream) {
  if (!plan) return SWIN3D_WATTN_EINVAL;
  const int64_t row = (int64_t)plan->desc.heads * plan->desc.head_dim;
  const swin3d_wattn_strides_t st = {row, row, row, row};
  return swin3d_wattn_run_strided(plan, q, k, v, o, &st, stream);
}

extern "C" int swin3d_adaln_residual(const swin3d_adaln_desc_t* d, const void* x, const void* res,
                                     const float* gamma, const float* beta, void* out, void* stream) {
  if (!d || !x || !res || !gamma || !beta || !out) return SWIN3D_WATTN_EINVAL;
  if (misaligned(x) || misaligned(res) || misaligned(gamma) || misaligned(beta) || misaligned(out))
    return SWIN3D_WATTN_EINVAL;
  auto known = [](int32_t t) { return t == SWIN3D_WATTN_F32 || t == SWIN3D_WATTN_BF16; };
  if (!known(d->x_dtype) || !known(d->res_dtype) || !known(d->out_dtype)) return SWIN3D_WATTN_EINVAL;
  if (d->rows <= 0 || d->B <= 0 || d->C <= 0) return SWIN3D_WATTN_EINVAL;
  if (!std::isfinite(d->eps) || !(d->eps > 0.0f)) return SWIN3D_WATTN_EINVAL;
  if (d->C % 256 != 0 || d->C > 4096) return SWIN3D_WATTN_EUNSUPPORTED;
  if (d->rows >= (int64_t(1) << 31) || d->rows * (int64_t)d->B >= (int64_t(1) << 31)) return SWIN3D_WATTN_EUNSUPPORTED;
  const int64_t n = d->rows * d->B * d->C;
  auto bytes = [n](int32_t t) { return n * (t == SWIN3D_WATTN_BF16 ? 2 : 4); };
  const int64_t xb = bytes(d->x_dtype), rb = bytes(d->res_dtype), ob = bytes(d->out_dtype);
  const int64_t pb = (int64_t)d->B * d->C * 4;
  if (overlaps(out, ob, x, xb) || overlaps(out, ob, gamma, pb) || overlaps(out, ob, beta, pb))
    return SWIN3D_WATTN_EINVAL;
  const bool in_place = out == res && d->out_dtype == d->res_dtype;
  if (!in_place && overlaps(out, ob, res, rb)) return SWIN3D_WATTN_EINVAL;
  return adaln_launch(d, x, res, gamma, beta, out, stream) == 0 ? SWIN3D_WATTN_OK : SWIN3D_WATTN_ELAUNCH;
}
