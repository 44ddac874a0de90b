// Swin3D shifted-window attention kernel, FP32 I/O, for gfx950 (MI355X).
//
// One workgroup computes one (window, head): it locates the window's tokens
// in grid layout with an integer index map (pad, cyclic shift and 3D window
// partition of the Flash-Aurora README, "Kernel fusion for backbone memory
// traffic"), gathers K and V into LDS and Q into registers, forms
// S = scale * Q K^T with the shifted-window bias and padding exclusion, takes
// the row softmax in FP32 and scatters O = softmax(S) V straight back to grid
// layout (inverse merge, unshift, crop). The whole window fits one LDS tile,
// so the softmax needs no cross-tile rescaling ("CuTe DSL window attention":
// single KV tile when the tile covers N).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "plan.h"

namespace {

struct Geom {
  int32_t X[3];      // real extents D, H, W
  int32_t P[3];      // padded extents
  int32_t win[3];    // window
  int32_t shift[3];  // cyclic shift
  int32_t nwin[3];   // windows per axis
  int32_t heads;
  int32_t N;         // tokens per window
  float scale;       // f32 kernel: natural-log units
  float bias;
  float c2;          // scale * log2(e)
  float bias2;       // cross-region bias * log2(e)
  int64_t sq, sk, sv, so;  // token strides of Q, K, V, O (elements)
};

constexpr uint32_t kPadCode = 0xFFu;

// Index map of one window slot. Slot n = (od, oh, ow) row-major inside window
// (kd, kh, kw); its shifted position is p = k * w + o, which holds grid
// position g = (p + s) mod P (p + s < 2P, so one conditional subtract).
// g >= X on any axis is padding. The region code has one bit per axis: set
// when that axis is shifted and p lies in the wrapped part [P - s, P).
__device__ __forceinline__ void slot_map(const Geom& g, int b, int kd, int kh, int kw, int n,
                                         int32_t& tok, uint32_t& code) {
  const int whw = g.win[1] * g.win[2];
  const int od = n / whw;
  const int r = n - od * whw;
  const int oh = r / g.win[2];
  const int ow = r - oh * g.win[2];
  const int p0 = kd * g.win[0] + od, p1 = kh * g.win[1] + oh, p2 = kw * g.win[2] + ow;
  int g0 = p0 + g.shift[0];
  if (g0 >= g.P[0]) g0 -= g.P[0];
  int g1 = p1 + g.shift[1];
  if (g1 >= g.P[1]) g1 -= g.P[1];
  int g2 = p2 + g.shift[2];
  if (g2 >= g.P[2]) g2 -= g.P[2];
  const bool valid = g0 < g.X[0] && g1 < g.X[1] && g2 < g.X[2];
  uint32_t c = 0;
  c |= (g.shift[0] > 0 && p0 >= g.P[0] - g.shift[0]) ? 1u : 0u;
  c |= (g.shift[1] > 0 && p1 >= g.P[1] - g.shift[1]) ? 2u : 0u;
  c |= (g.shift[2] > 0 && p2 >= g.P[2] - g.shift[2]) ? 4u : 0u;
  code = valid ? c : kPadCode;
  tok = valid ? ((b * g.X[0] + g0) * g.X[1] + g1) * g.X[2] + g2 : -1;
}

// blockIdx.x = window * heads + head, windows numbered (b, kd, kh, kw) row-major:
// neighbouring workgroups read the other heads of the same tokens.
__device__ __forceinline__ void decode_item(const Geom& g, int item, int& b, int& kd, int& kh,
                                            int& kw, int& head) {
  head = item % g.heads;
  int w = item / g.heads;
  const int per_b = g.nwin[0] * g.nwin[1] * g.nwin[2];
  b = w / per_b;
  w -= b * per_b;
  kd = w / (g.nwin[1] * g.nwin[2]);
  w -= kd * (g.nwin[1] * g.nwin[2]);
  kh = w / g.nwin[2];
  kw = w - kh * g.nwin[2];
}

// ---------------------------------------------------------------------------
// FP32 path: vector-ALU kernel, one thread per query slot. K and V of the
// window sit in LDS; every thread reads the same key row at the same time
// (an LDS broadcast). Two passes over the keys: row max, then exp / sum / PV.
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void wattn_f32_kernel(const float* __restrict__ q,
                                                        const float* __restrict__ k,
                                                        const float* __restrict__ v,
                                                        float* __restrict__ o, Geom g) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* Ks = reinterpret_cast<float*>(smem);
  float* Vs = Ks + g.N * DH;
  int32_t* tokS = reinterpret_cast<int32_t*>(Vs + g.N * DH);
  uint32_t* codeS = reinterpret_cast<uint32_t*>(tokS + g.N);

  int b, kd, kh, kw, head;
  decode_item(g, blockIdx.x, b, kd, kh, kw, head);
  const int tid = threadIdx.x;
  for (int n = tid; n < g.N; n += blockDim.x) {
    int32_t t;
    uint32_t c;
    slot_map(g, b, kd, kh, kw, n, t, c);
    tokS[n] = t;
    codeS[n] = c;
  }
  __syncthreads();

  const size_t hoff = (size_t)head * DH;
  constexpr int C = DH / 4;
  for (int idx = tid; idx < g.N * C; idx += blockDim.x) {
    const int n = idx / C, c = idx - n * C;
    const int32_t t = tokS[n];
    float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
    if (t >= 0) {
      kk = *reinterpret_cast<const float4*>(k + (size_t)t * g.sk + hoff + 4 * c);
      vv = *reinterpret_cast<const float4*>(v + (size_t)t * g.sv + hoff + 4 * c);
    }
    *reinterpret_cast<float4*>(Ks + n * DH + 4 * c) = kk;
    *reinterpret_cast<float4*>(Vs + n * DH + 4 * c) = vv;
  }
  __syncthreads();

  const int n = tid;
  if (n >= g.N) return;
  const int32_t t = tokS[n];
  if (t < 0) return;  // padding query: cropped, never written
  const uint32_t cq = codeS[n];
  const size_t qoff = (size_t)t * g.sq + hoff;
  const size_t ooff = (size_t)t * g.so + hoff;

  float qr[DH];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const float4 x = *reinterpret_cast<const float4*>(q + qoff + 4 * c);
    qr[4 * c] = x.x;
    qr[4 * c + 1] = x.y;
    qr[4 * c + 2] = x.z;
    qr[4 * c + 3] = x.w;
  }

  auto logit = [&](int j) -> float {
    const float* kr = Ks + j * DH;
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float4 x = *reinterpret_cast<const float4*>(kr + 4 * c);
      s = fmaf(qr[4 * c], x.x, s);
      s = fmaf(qr[4 * c + 1], x.y, s);
      s = fmaf(qr[4 * c + 2], x.z, s);
      s = fmaf(qr[4 * c + 3], x.w, s);
    }
    const uint32_t ck = codeS[j];
    const float add = (ck == kPadCode) ? -INFINITY : (ck != cq ? g.bias : 0.f);
    return fmaf(s, g.scale, add);
  };

  float m = -INFINITY;
  for (int j = 0; j < g.N; ++j) m = fmaxf(m, logit(j));

  float acc[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) acc[d] = 0.f;
  float l = 0.f;
  for (int j = 0; j < g.N; ++j) {
    const float p = expf(logit(j) - m);
    l += p;
    const float* vr = Vs + j * DH;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float4 x = *reinterpret_cast<const float4*>(vr + 4 * c);
      acc[4 * c] = fmaf(p, x.x, acc[4 * c]);
      acc[4 * c + 1] = fmaf(p, x.y, acc[4 * c + 1]);
      acc[4 * c + 2] = fmaf(p, x.z, acc[4 * c + 2]);
      acc[4 * c + 3] = fmaf(p, x.w, acc[4 * c + 3]);
    }
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    *reinterpret_cast<float4*>(o + ooff + 4 * c) =
        make_float4(acc[4 * c] * inv, acc[4 * c + 1] * inv, acc[4 * c + 2] * inv, acc[4 * c + 3] * inv);
  }
}

Geom make_geom(const swin3d_wattn_plan* p, const swin3d_wattn_strides_t* st) {
  Geom g;
  const swin3d_wattn_desc_t& d = p->desc;
  g.X[0] = d.D;
  g.X[1] = d.H;
  g.X[2] = d.W;
  for (int a = 0; a < 3; ++a) {
    g.P[a] = p->padded[a];
    g.win[a] = d.window[a];
    g.shift[a] = d.shift[a];
    g.nwin[a] = p->nwin[a];
  }
  g.heads = d.heads;
  g.N = p->N;
  g.scale = d.scale;
  g.bias = d.cross_region_bias;
  g.c2 = p->c2;
  g.bias2 = p->bias2;
  g.sq = st->q;
  g.sk = st->k;
  g.sv = st->v;
  g.so = st->o;
  return g;
}

size_t f32_lds_bytes(int N, int dh) { return (size_t)N * dh * 4 * 2 + (size_t)N * 8; }

template <int DH>
hipError_t launch(const swin3d_wattn_plan* p, const void* q, const void* k, const void* v, void* o,
                  const swin3d_wattn_strides_t* st, hipStream_t s) {
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&wattn_f32_kernel<DH>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)f32_lds_bytes(256, DH));
  });
  if (attr_err != hipSuccess) return attr_err;
  Geom g = make_geom(p, st);
  const float* qq = static_cast<const float*>(q);
  const float* kk = static_cast<const float*>(k);
  const float* vv = static_cast<const float*>(v);
  float* oo = static_cast<float*>(o);
  void* args[] = {&qq, &kk, &vv, &oo, &g};
  return hipLaunchKernel(reinterpret_cast<const void*>(&wattn_f32_kernel<DH>), dim3((unsigned)p->workgroups),
                         dim3(p->threads), args, f32_lds_bytes(p->N, DH), s);
}

}  // namespace

int wattn_launch_f32(const swin3d_wattn_plan* p, const void* q, const void* k, const void* v, void* o,
                     const swin3d_wattn_strides_t* stride, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = p->desc.head_dim == 32 ? launch<32>(p, q, k, v, o, stride, s)
                                              : launch<64>(p, q, k, v, o, stride, s);
  return (int)e;
}
