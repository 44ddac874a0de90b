// Swin3D shifted-window attention kernels for gfx950 (MI355X).
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
  float c2;          // bf16 kernel: scale * log2(e)
  float bias2;       // cross-region bias * log2(e)
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

  const size_t RS = (size_t)g.heads * DH;
  const size_t hoff = (size_t)head * DH;
  constexpr int C = DH / 4;
  for (int idx = tid; idx < g.N * C; idx += blockDim.x) {
    const int n = idx / C, c = idx - n * C;
    const int32_t t = tokS[n];
    float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
    if (t >= 0) {
      const size_t off = (size_t)t * RS + hoff + 4 * c;
      kk = *reinterpret_cast<const float4*>(k + off);
      vv = *reinterpret_cast<const float4*>(v + off);
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
  const size_t qoff = (size_t)t * RS + hoff;

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
    *reinterpret_cast<float4*>(o + qoff + 4 * c) =
        make_float4(acc[4 * c] * inv, acc[4 * c + 1] * inv, acc[4 * c + 2] * inv, acc[4 * c + 3] * inv);
  }
}

// ---------------------------------------------------------------------------
// BF16 path: matrix-core kernel for N = 144 (window (2, 6, 12)), head_dim 64.
//
// Orientation. The kernel computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16
// (A = 16 keys x 32 dims from LDS, B = 32 dims x 16 queries from registers).
// Its accumulator gives each lane four keys of one query, which is exactly
// the layout the B operand of the next product wants, so O^T = V^T P^T runs
// from registers with no LDS round trip for P: for key step j the lane packs
// keys {32j + 4g + i} and {32j + 16 + 4g + i} (g = lane / 16, i = 0..3), and
// reads V^T with the same key assignment. The 144 keys are four 32-key
// steps plus one 16-key step (v_mfma_f32_16x16x16_bf16).
//
// Work split: 3 waves x 3 query tiles of 16 rows = 144 queries.
// LDS: K row-major [144][72] (64 + 8 pad), V^T [64][152] (144 + 8 pad),
// slot table (token index, region code). The softmax is FP32 in the log2
// domain: t = S * scale * log2(e) + bias * log2(e), p = 2^(t - max t).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef short short4_t __attribute__((__vector_size__(8)));
typedef __bf16 bf16x4_t __attribute__((__vector_size__(8)));
typedef float floatx4 __attribute__((__vector_size__(16)));
typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
typedef uint32_t u32x2 __attribute__((__vector_size__(8)));

// Matrix-core ordering. An MFMA whose accumulator input comes from one of
// the last few MFMAs waits inside the matrix pipeline after issue and reads
// its A/B registers late; an LDS load issued behind it can overwrite them
// first. The kernels therefore interleave independent accumulators and pin
// the MFMA order with a scheduling barrier that every other instruction
// class (VALU, SALU, LDS, VMEM, transcendental) may still cross.
#define WATTN_PIN_MFMA() __builtin_amdgcn_sched_barrier(0x7F6)

constexpr int kN = 144;
constexpr int kNT = 9;           // key / query tiles of 16
constexpr int kDH = 64;
constexpr int kWaves = 3;
constexpr int kQTPerWave = 3;
constexpr int kThreads = kWaves * 64;
constexpr int kKStride = 72;     // bf16 per K row in LDS
constexpr int kVStride = 152;    // bf16 per V^T row in LDS

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// d-row of V^T that A-operand row m of output tile t reads. Chosen so the
// accumulator of tiles (0, 1) gives each lane dims [8g, 8g + 8) and tiles
// (2, 3) dims [32 + 8g, 32 + 8g + 8): two contiguous 16-byte stores per lane.
__device__ __forceinline__ int dmap(int t, int m) {
  return (t >> 1) * 32 + (m >> 2) * 8 + (t & 1) * 4 + (m & 3);
}

__device__ __forceinline__ float wave_max16x4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum16x4(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void wattn_bf16_n144_d64(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ k,
                                                               const uint16_t* __restrict__ v,
                                                               uint16_t* __restrict__ o, Geom g) {
  __shared__ __align__(16) uint16_t Ks[kN * kKStride];
  __shared__ __align__(16) uint16_t Vt[kDH * kVStride];
  __shared__ int32_t tokS[kN];
  __shared__ __align__(16) uint8_t codeS[kN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;

  int b, kd, kh, kw, head;
  decode_item(g, blockIdx.x, b, kd, kh, kw, head);

  int need_mask = 0;
  if (tid < kN) {
    int32_t t;
    uint32_t c;
    slot_map(g, b, kd, kh, kw, tid, t, c);
    tokS[tid] = t;
    codeS[tid] = (uint8_t)c;
    need_mask = c != 0;
  }
  need_mask = __syncthreads_or(need_mask);

  const size_t RS = (size_t)g.heads * kDH;
  const size_t hoff = (size_t)head * kDH;

  // ---- issue every global load of this (window, head) before any use ----
  u32x4 kreg[6];
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const int c = tid + kThreads * i;
    const int row = c >> 3, part = c & 7;
    const int32_t t = tokS[row];
    kreg[i] = t >= 0 ? load16(k + (size_t)t * RS + hoff + part * 8) : u32x4{0, 0, 0, 0};
  }
  u32x4 va[3], vb[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int c = tid + kThreads * i;
    const int pr = c >> 3, part = c & 7;
    const int32_t t0 = tokS[2 * pr], t1 = tokS[2 * pr + 1];
    va[i] = t0 >= 0 ? load16(v + (size_t)t0 * RS + hoff + part * 8) : u32x4{0, 0, 0, 0};
    vb[i] = t1 >= 0 ? load16(v + (size_t)t1 * RS + hoff + part * 8) : u32x4{0, 0, 0, 0};
  }
  u32x4 qreg[kQTPerWave][2];
#pragma unroll
  for (int qi = 0; qi < kQTPerWave; ++qi) {
    const int row = (wave * kQTPerWave + qi) * 16 + l16;
    const int32_t t = tokS[row];
#pragma unroll
    for (int s = 0; s < 2; ++s)
      qreg[qi][s] = t >= 0 ? load16(q + (size_t)t * RS + hoff + 32 * s + 8 * g4) : u32x4{0, 0, 0, 0};
  }

  // ---- K row-major into LDS; V transposed (pairs of keys per 32-bit write) ----
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const int c = tid + kThreads * i;
    const int row = c >> 3, part = c & 7;
    *reinterpret_cast<u32x4*>(&Ks[row * kKStride + part * 8]) = kreg[i];
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int c = tid + kThreads * i;
    const int pr = c >> 3, part = c & 7;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t a = va[i][j >> 1], bb = vb[i][j >> 1];
      const uint32_t packed = (j & 1) ? ((a >> 16) | (bb & 0xFFFF0000u)) : ((a & 0xFFFFu) | (bb << 16));
      *reinterpret_cast<uint32_t*>(&Vt[(part * 8 + j) * kVStride + 2 * pr]) = packed;
    }
  }
  __syncthreads();

  const float c2 = g.c2;
#pragma unroll
  for (int qi = 0; qi < kQTPerWave; ++qi) {
    const int qt = wave * kQTPerWave + qi;
    // Consecutive MFMAs stay independent: the dims step is the outer loop.
    floatx4 S[kNT];
#pragma unroll
    for (int kt = 0; kt < kNT; ++kt) S[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&Ks[(kt * 16 + l16) * kKStride + 32 * s + 8 * g4]);
        S[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, qreg[qi][s]), S[kt], 0, 0, 0);
        WATTN_PIN_MFMA();
      }
    }

    float mx = -INFINITY;
    if (!need_mask) {
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, S[kt][i]);
      mx = wave_max16x4(mx);
      const float nm = -mx * c2;
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[kt][i] = __builtin_amdgcn_exp2f(fmaf(S[kt][i], c2, nm));
    } else {
      const uint32_t cq = codeS[qt * 16 + l16];
      const float bias2 = g.bias2;
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt) {
        const uint32_t c4 = *reinterpret_cast<const uint32_t*>(&codeS[kt * 16 + 4 * g4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t ck = (c4 >> (8 * i)) & 0xFFu;
          float add = ck == cq ? 0.f : bias2;
          add = ck == kPadCode ? -INFINITY : add;
          const float x = fmaf(S[kt][i], c2, add);
          S[kt][i] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = wave_max16x4(mx);
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[kt][i] = __builtin_amdgcn_exp2f(S[kt][i] - mx);
    }
    float sum = 0.f;
#pragma unroll
    for (int kt = 0; kt < kNT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sum += S[kt][i];
    sum = wave_sum16x4(sum);
    const float inv = 1.0f / sum;

    bf16x8_t Pb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Pb[j][i] = (__bf16)S[2 * j][i];
        Pb[j][4 + i] = (__bf16)S[2 * j + 1][i];
      }
    }
    bf16x4_t Pt;
#pragma unroll
    for (int i = 0; i < 4; ++i) Pt[i] = (__bf16)S[8][i];

    // Four independent accumulators, key step outer; the 16-key tail goes
    // first so it never waits on a fresh accumulator.
    floatx4 O[4];
    const uint16_t* vrow[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      vrow[t] = &Vt[dmap(t, l16) * kVStride];
      const short4_t a4 = *reinterpret_cast<const short4_t*>(vrow[t] + 128 + 4 * g4);
      O[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a4, __builtin_bit_cast(short4_t, Pt),
                                                       floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      WATTN_PIN_MFMA();
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow[t] + 32 * j + 4 * g4);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow[t] + 32 * j + 16 + 4 * g4);
        const u32x4 a = u32x4{lo[0], lo[1], hi[0], hi[1]};
        O[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), Pb[j], O[t], 0, 0, 0);
        WATTN_PIN_MFMA();
      }
    }

    const int32_t t = tokS[qt * 16 + l16];
    if (t >= 0) {
      uint16_t* out = o + (size_t)t * RS + hoff;
      bf16x8_t r0, r1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        r0[i] = (__bf16)(O[0][i] * inv);
        r0[4 + i] = (__bf16)(O[1][i] * inv);
        r1[i] = (__bf16)(O[2][i] * inv);
        r1[4 + i] = (__bf16)(O[3][i] * inv);
      }
      *reinterpret_cast<bf16x8_t*>(out + 8 * g4) = r0;
      *reinterpret_cast<bf16x8_t*>(out + 32 + 8 * g4) = r1;
    }
  }
}

Geom make_geom(const swin3d_wattn_plan* p) {
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
  return g;
}

size_t f32_lds_bytes(int N, int dh) { return (size_t)N * dh * 4 * 2 + (size_t)N * 8; }

template <int DH>
hipError_t launch_f32(const swin3d_wattn_plan* p, const void* q, const void* k, const void* v, void* o,
                      hipStream_t s) {
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&wattn_f32_kernel<DH>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)f32_lds_bytes(256, DH));
  });
  if (attr_err != hipSuccess) return attr_err;
  Geom g = make_geom(p);
  const float* qq = static_cast<const float*>(q);
  const float* kk = static_cast<const float*>(k);
  const float* vv = static_cast<const float*>(v);
  float* oo = static_cast<float*>(o);
  void* args[] = {&qq, &kk, &vv, &oo, &g};
  return hipLaunchKernel(reinterpret_cast<const void*>(&wattn_f32_kernel<DH>), dim3((unsigned)p->workgroups),
                         dim3(p->threads), args, f32_lds_bytes(p->N, DH), s);
}

}  // namespace

int swin3d_wattn_launch(const swin3d_wattn_plan* p, const void* q, const void* k, const void* v, void* o,
                        void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (p->kernel == 1) {
    Geom g = make_geom(p);
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    const uint16_t* vv = static_cast<const uint16_t*>(v);
    uint16_t* oo = static_cast<uint16_t*>(o);
    void* args[] = {&qq, &kk, &vv, &oo, &g};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&wattn_bf16_n144_d64), dim3((unsigned)p->workgroups),
                        dim3(kThreads), args, 0, s);
  } else if (p->desc.head_dim == 32) {
    e = launch_f32<32>(p, q, k, v, o, s);
  } else {
    e = launch_f32<64>(p, q, k, v, o, s);
  }
  return e == hipSuccess ? SWIN3D_WATTN_OK : SWIN3D_WATTN_ELAUNCH;
}
