// Fused AdaLN + residual for gfx950 (MI355X): the step around each Swin3D
// attention block that the Flash-Aurora README fuses ("Kernel fusion for
// backbone memory traffic": LayerNorm, FiLM modulation and the residual add
// without a full-width intermediate, optionally emitting FP32 activations
// between blocks).
//
// For token row t of batch element b (C channels):
//   xhat = (x - mean) / sqrt(var + eps)      (biased variance over C)
//   out  = res + gamma[b] * xhat + beta[b]
// x, res and out are each bf16 or fp32; gamma, beta are fp32 [B, C]. All
// arithmetic is FP32.
//
// One wave per row: the row stays in registers (two passes over registers,
// not over memory), so the kernel reads x and res once and writes out once.
// Lane l handles the 4-channel units l, l + 64, ..., so every load and store
// instruction of a wave covers a contiguous span of the row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.h"
#include "plan.h"

namespace {

typedef float floatx4 __attribute__((__vector_size__(16)));
typedef __bf16 bf16x4_t __attribute__((__vector_size__(8)));
typedef uint32_t u32x2 __attribute__((__vector_size__(8)));

constexpr int kWaves = 4;
constexpr int kMaxUnits = 16;  // C <= 64 lanes x 16 units x 4 channels = 4096

using fastdiv::FastDiv;
using fastdiv::fdiv;
using fastdiv::make_fastdiv;

struct AdalnParams {
  int32_t rows;   // B * T
  int32_t row0;   // first row of this launch
  int32_t C;
  int32_t units;  // C / 256: 4-channel units per lane
  FastDiv div_t;  // by T (rows per batch element)
  float eps;
  float inv_c;
};

// 4 channels in, as fp32 (non-temporal: x and res are read once)
__device__ __forceinline__ floatx4 load4(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
}
__device__ __forceinline__ floatx4 load4(const __bf16* p) {
  const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return __builtin_convertvector(__builtin_bit_cast(bf16x4_t, w), floatx4);
}
// 4 channels out (bf16: round to nearest even, whole-vector conversion),
// non-temporal: the output is written once and read by the next kernel
// (measured 3.6% faster than ordinary stores at the stage-1 token count)
__device__ __forceinline__ void store4(float* p, floatx4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<floatx4*>(p));
}
__device__ __forceinline__ void store4(__bf16* p, floatx4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x2, __builtin_convertvector(v, bf16x4_t)),
                              reinterpret_cast<u32x2*>(p));
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// U: 4-channel units per lane. U < kMaxUnits is exact (C = 256 U, the common
// widths); U = kMaxUnits serves every other width, each unit guarded by
// i < units. For U <= 4 every load of the row (x, res, gamma, beta) is issued
// up front, so a wave makes one memory round trip before its stores; larger
// rows load res, gamma and beta after the statistics to stay within the
// register budget.
template <typename XT, typename RT, typename OT, int U>
__global__ __launch_bounds__(64 * kWaves) void adaln_residual_kernel(const XT* __restrict__ x, const RT* res,
                                                                      const float* __restrict__ gamma,
                                                                      const float* __restrict__ beta, OT* out,
                                                                      const AdalnParams p) {
  constexpr bool kEarly = U <= 4;
  constexpr bool kGuard = U == kMaxUnits;
  const int lane = threadIdx.x & 63;
  const int row = p.row0 + (int)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= p.rows) return;  // whole waves only
  const int b = (int)fdiv((uint32_t)row, p.div_t);
  const size_t base = (size_t)row * p.C;
  const float* g = gamma + (size_t)b * p.C;
  const float* be = beta + (size_t)b * p.C;

  floatx4 v[U], r[kEarly ? U : 1], gg[kEarly ? U : 1], bb[kEarly ? U : 1];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < U; ++i) {
    if (!kGuard || i < p.units) {
      const int c = 4 * (lane + 64 * i);
      v[i] = load4(x + base + c);
      if constexpr (kEarly) {
        r[i] = load4(res + base + c);
        gg[i] = *reinterpret_cast<const floatx4*>(g + c);
        bb[i] = *reinterpret_cast<const floatx4*>(be + c);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < U; ++i)
    if (!kGuard || i < p.units) s += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
  const float mean = wave_sum(s) * p.inv_c;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < U; ++i) {
    if (!kGuard || i < p.units) {
      const floatx4 d = v[i] - mean;
      v[i] = d;
      q += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) * p.inv_c + p.eps);

#pragma unroll
  for (int i = 0; i < U; ++i) {
    if (!kGuard || i < p.units) {
      const int c = 4 * (lane + 64 * i);
      if constexpr (kEarly) {
        store4(out + base + c, r[i] + gg[i] * (v[i] * rstd) + bb[i]);
      } else {
        const floatx4 g4 = *reinterpret_cast<const floatx4*>(g + c);
        const floatx4 b4 = *reinterpret_cast<const floatx4*>(be + c);
        store4(out + base + c, load4(res + base + c) + g4 * (v[i] * rstd) + b4);
      }
    }
  }
}

template <typename XT, typename RT, typename OT, int U>
hipError_t launch_u(const swin3d_adaln_desc_t* d, const void* x, const void* res, const float* gamma,
                    const float* beta, void* out, hipStream_t s) {
  AdalnParams p;
  p.rows = (int32_t)(d->rows * d->B);
  p.C = d->C;
  p.units = d->C / 256;
  p.div_t = make_fastdiv((uint32_t)d->rows);
  p.eps = d->eps;
  p.inv_c = 1.0f / (float)d->C;
  const XT* xx = static_cast<const XT*>(x);
  const RT* rr = static_cast<const RT*>(res);
  OT* oo = static_cast<OT*>(out);
  void* args[] = {&xx, &rr, &gamma, &beta, &oo, &p};
  // a dispatch counts its work-items in 32 bits: at most kPiece rows (2^30
  // work-items) per launch, in order on the stream
  constexpr int32_t kPiece = 1 << 24;
  for (p.row0 = 0; p.row0 < p.rows; p.row0 += kPiece) {
    const int32_t n = p.rows - p.row0 < kPiece ? p.rows - p.row0 : kPiece;
    const unsigned blocks = (unsigned)((n + kWaves - 1) / kWaves);
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&adaln_residual_kernel<XT, RT, OT, U>),
                                         dim3(blocks), dim3(64 * kWaves), args, 0, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename XT, typename RT, typename OT>
hipError_t launch_t(const swin3d_adaln_desc_t* d, const void* x, const void* res, const float* gamma,
                    const float* beta, void* out, hipStream_t s) {
  switch (d->C / 256) {  // 1..16, checked on the host
    case 1: return launch_u<XT, RT, OT, 1>(d, x, res, gamma, beta, out, s);
    case 2: return launch_u<XT, RT, OT, 2>(d, x, res, gamma, beta, out, s);
    case 4: return launch_u<XT, RT, OT, 4>(d, x, res, gamma, beta, out, s);
    case 8: return launch_u<XT, RT, OT, 8>(d, x, res, gamma, beta, out, s);
    default: return launch_u<XT, RT, OT, kMaxUnits>(d, x, res, gamma, beta, out, s);
  }
}

template <typename XT, typename RT>
hipError_t launch_o(const swin3d_adaln_desc_t* d, const void* x, const void* res, const float* gamma,
                    const float* beta, void* out, hipStream_t s) {
  return d->out_dtype == SWIN3D_WATTN_BF16 ? launch_t<XT, RT, __bf16>(d, x, res, gamma, beta, out, s)
                                           : launch_t<XT, RT, float>(d, x, res, gamma, beta, out, s);
}

template <typename XT>
hipError_t launch_r(const swin3d_adaln_desc_t* d, const void* x, const void* res, const float* gamma,
                    const float* beta, void* out, hipStream_t s) {
  return d->res_dtype == SWIN3D_WATTN_BF16 ? launch_o<XT, __bf16>(d, x, res, gamma, beta, out, s)
                                           : launch_o<XT, float>(d, x, res, gamma, beta, out, s);
}

}  // namespace

int adaln_launch(const swin3d_adaln_desc_t* d, const void* x, const void* res, const float* gamma,
                 const float* beta, void* out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = d->x_dtype == SWIN3D_WATTN_BF16 ? launch_r<__bf16>(d, x, res, gamma, beta, out, s)
                                                       : launch_r<float>(d, x, res, gamma, beta, out, s);
  return (int)e;
}
