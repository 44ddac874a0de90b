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
// BF16 path: matrix-core kernel for N = 144 tokens per window (window
// (2, 6, 12) or any other with 144 slots) and head_dim 64.
//
// Work: one workgroup of four waves per (window, head) item, dispatched
// head-major (item = head * n_windows + window): the workgroups in flight
// read one head of many neighbouring windows, the order HBM serves best for
// these 128-byte rows. Small workgroups (38 KB of LDS, <= 128 VGPRs) let four
// of them share a CU, so one workgroup's loads overlap another's math.
//
// LDS: K and V row-major (128 B rows, 16-byte chunks XOR-swizzled by row
// bits 1..3 so that every operand read below hits distinct bank groups),
// the slot table (token index, region code) and a small mask-feature table.
// Each wave loads the Q operands of its own query tiles into registers.
//
// S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = 16 keys x 32 dims, B = 32
// dims x 16 queries). Its accumulator gives each lane four keys of one
// query, which is the B-operand layout of O^T = V^T P^T, so P never leaves
// registers. The V^T operand is read straight from row-major V with
// ds_read_b64_tr_b16: within each 16-lane group, input lane 4e + q points at
// 4 dims of key e and output lane m receives key e of dim 4(m/4) + m%4.
//
// Mask on the matrix core: a third k-step of 32 extra "dims" adds the
// shifted-window bias. Q gets a one-hot of its region in each of three
// 8-wide slots (plus a constant 1 in a pad column); K gets bias/scale (split
// into three bf16 terms) at every region other than its own, and -2^100 in
// the pad column when it is padding. The product adds exactly the bias
// where regions differ and pushes padding keys to a zero weight. A key's
// features depend only on its region code, so they come from a table.
// Row sums of P come from the matrix core too: a fifth accumulator whose A
// operand is all ones, so the normaliser sums the same bf16 P as the output.
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
// first. The kernel therefore interleaves independent accumulators and pins
// the MFMA order with a scheduling barrier that every other instruction
// class (VALU, SALU, LDS, VMEM, transcendental) may still cross.
#define WATTN_PIN_MFMA() __builtin_amdgcn_sched_barrier(0x7F6)
// The same, but LDS instructions stay in place too: used where the source
// issues LDS reads a fixed distance ahead of the MFMAs that consume them.
#define WATTN_PIN_MFMA_LDS() __builtin_amdgcn_sched_barrier(0x676)

constexpr int kN = 144;
constexpr int kNT = 9;                    // key / query tiles of 16
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxQT = (kNT + kWaves - 1) / kWaves;  // query tiles per wave (at most)
constexpr int kTensorBytes = kN * 128;    // one 144 x 64 bf16 tile
// LDS layout (bytes): K tile, V tile, mask-feature table (9 codes x 4
// groups x 16 B; code 8 = padding), region code and token of each slot
constexpr int kXtOff = 2 * kTensorBytes;
constexpr int kCodeOff = kXtOff + 9 * 4 * 16;
constexpr int kTokOff = kCodeOff + kN;
constexpr int kSmemBytes = kTokOff + kN * 4;

struct AttnParams {
  int32_t X[3], P[3], shift[3], win[3], nwin[3];
  int32_t special[3][3];
  int32_t heads;
  int32_t n_items;
  float c2;
  uint32_t beta01;  // bf16 beta term 0 | term 1 << 16
  uint32_t beta2;   // bf16 beta term 2
  uint32_t pad;     // bf16 padding-key offset
  uint32_t slot[kN];
};

__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 1) | (((r >> 3) & 1) << 1) | (((r >> 2) & 1) << 2); }
// byte offset of 16-byte chunk c (0..7) of row r in a 128-byte-row tensor tile
__device__ __forceinline__ int qkv_off(int r, int c) { return r * 128 + ((c ^ swz(r)) << 4); }
// first dim of the 4-dim group q (0..3) held by output tile t (0..3); the
// alternation of the +4 between neighbouring groups makes each transposed
// read touch both 8-byte halves of the 16-byte chunks it spans
__device__ __forceinline__ int dbase(int t, int q) { return (t >> 1) * 32 + q * 8 + 4 * ((q ^ t) & 1); }

__device__ __forceinline__ float wave_max16x4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

struct WinPos {
  int b, k[3];
  bool masked;
};

// Window w (batch folded in) -> (b, kd, kh, kw) and whether it needs the
// mask path (a region cut or padding along some axis).
__device__ __forceinline__ WinPos decode_window(const AttnParams& p, int w) {
  WinPos it;
  const int per_b = p.nwin[0] * p.nwin[1] * p.nwin[2];
  it.b = w / per_b;
  w -= it.b * per_b;
  it.k[0] = w / (p.nwin[1] * p.nwin[2]);
  w -= it.k[0] * (p.nwin[1] * p.nwin[2]);
  it.k[1] = w / p.nwin[2];
  it.k[2] = w - it.k[1] * p.nwin[2];
  bool m = false;
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int j = 0; j < 3; ++j) m |= p.special[a][j] == it.k[a];
  it.masked = m;
  return it;
}

// Grid position of slot (od, oh, ow) of a window: token index, or -1 for
// padding, and the region code (one bit per axis: shifted axis and position
// in the wrapped part [P - s, P)).
__device__ __forceinline__ void map_slot(const AttnParams& p, const WinPos& it, uint32_t packed, int32_t& tok,
                                         uint32_t& code) {
  const int o[3] = {(int)(packed & 0xFF), (int)((packed >> 8) & 0xFF), (int)(packed >> 16)};
  int g[3];
  uint32_t c = 0;
  bool valid = true;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    const int pa = it.k[a] * p.win[a] + o[a];
    int ga = pa + p.shift[a];
    ga = ga >= p.P[a] ? ga - p.P[a] : ga;
    g[a] = ga;
    valid = valid && ga < p.X[a];
    c |= (p.shift[a] > 0 && pa >= p.P[a] - p.shift[a]) ? (1u << a) : 0u;
  }
  tok = valid ? ((it.b * p.X[0] + g[0]) * p.X[1] + g[1]) * p.X[2] + g[2] : -1;
  code = valid ? c : kPadCode;
}

__device__ __forceinline__ u32x4 ldg16(const uint16_t* ptr) { return *reinterpret_cast<const u32x4*>(ptr); }

__device__ __forceinline__ short4_t lds_tr(const uint8_t* smem, int byte_off) {
  typedef short4_t __attribute__((address_space(3))) * lds_ptr;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(smem + byte_off));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((__vector_size__(4)));
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void wattn_bf16_item(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, const AttnParams p) {
  __shared__ __align__(16) uint8_t smem[kSmemBytes];
  uint8_t* codeS = smem + kCodeOff;
  int32_t* tokS = reinterpret_cast<int32_t*>(smem + kTokOff);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  const int heads = p.heads;
  const size_t RS = (size_t)heads * 64;
  const int n_windows = p.n_items / heads;
  const int item = blockIdx.x;
  const int head = item / n_windows;
  const int win = item - head * n_windows;
  const WinPos cur = decode_window(p, win);
  const size_t hoff = (size_t)head * 64;

  // ---- slot table of the window ----
  uint32_t mycode = kPadCode;
  for (int r = tid; r < kN; r += kThreads) {
    int32_t t;
    map_slot(p, cur, p.slot[r], t, mycode);
    tokS[r] = t;
    codeS[r] = (uint8_t)mycode;
  }
  __syncthreads();

  // ---- gather: K and V rows into registers, Q operands of this wave's tiles ----
  constexpr int kChunks = kN * 8;
  constexpr int kPer = (kChunks + kThreads - 1) / kThreads;
  u32x4 kr[kPer], vr[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int c = tid + kThreads * j;
    kr[j] = vr[j] = u32x4{0, 0, 0, 0};
    if (c < kChunks) {
      const int32_t t = tokS[c >> 3];
      if (t >= 0) {
        const size_t off = (size_t)t * RS + hoff + (c & 7) * 8;
        kr[j] = ldg16(k + off);
        vr[j] = ldg16(v + off);
      }
    }
  }
  u32x4 qr[kMaxQT][2];
#pragma unroll
  for (int qi = 0; qi < kMaxQT; ++qi) {
    const int qt = wave + kWaves * qi;
    qr[qi][0] = qr[qi][1] = u32x4{0, 0, 0, 0};
    if (qt < kNT) {
      const int32_t t = tokS[qt * 16 + l16];
      if (t >= 0) {
        const size_t off = (size_t)t * RS + hoff + 8 * g4;
        qr[qi][0] = ldg16(q + off);
        qr[qi][1] = ldg16(q + off + 32);
      }
    }
  }
  // mask-feature table (only windows with a cut or padding use it)
  if (cur.masked && tid < 36) {
    const uint32_t beta[3] = {p.beta01 & 0xFFFFu, p.beta01 >> 16, p.beta2 & 0xFFFFu};
    const uint32_t ck = tid >> 2, part = tid & 3;  // ck == 8: padding key
    u32x4 w = u32x4{0, 0, 0, 0};
    if (ck == 8) {
      if (part == 3) w[0] = p.pad;
    } else if (part < 3) {
      const uint32_t bt = beta[part];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (uint32_t)(2 * e) != ck ? bt : 0u;
        const uint32_t hi = (uint32_t)(2 * e + 1) != ck ? bt : 0u;
        w[e] = lo | (hi << 16);
      }
    }
    *reinterpret_cast<u32x4*>(smem + kXtOff + tid * 16) = w;
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int c = tid + kThreads * j;
    if (c < kChunks) {
      *reinterpret_cast<u32x4*>(smem + qkv_off(c >> 3, c & 7)) = kr[j];
      *reinterpret_cast<u32x4*>(smem + kTensorBytes + qkv_off(c >> 3, c & 7)) = vr[j];
    }
  }
  __syncthreads();

  const float c2 = p.c2;
  const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
  for (int qi = 0; qi < kMaxQT; ++qi) {
    const int qt = wave + kWaves * qi;
    if (qt >= kNT) break;
    const bf16x8_t qop[2] = {__builtin_bit_cast(bf16x8_t, qr[qi][0]), __builtin_bit_cast(bf16x8_t, qr[qi][1])};

    floatx4 S[kNT];
#pragma unroll
    for (int kt = 0; kt < kNT; ++kt) S[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
    {
      constexpr int kAhead = 8;
      bf16x8_t kf[2 * kNT];
      auto kread = [&](int idx) {
        const int s = idx / kNT, kt = idx % kNT;
        kf[idx] = *reinterpret_cast<const bf16x8_t*>(smem + qkv_off(kt * 16 + l16, 4 * s + g4));
      };
#pragma unroll
      for (int idx = 0; idx < kAhead; ++idx) kread(idx);
#pragma unroll
      for (int idx = 0; idx < 2 * kNT; ++idx) {
        const int s = idx / kNT, kt = idx % kNT;
        S[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[idx], qop[s], S[kt], 0, 0, 0);
        WATTN_PIN_MFMA_LDS();
        if (idx + kAhead < 2 * kNT) kread(idx + kAhead);
      }
    }
    if (cur.masked) {
      const uint32_t cq = codeS[qt * 16 + l16];
      u32x4 qx = u32x4{0, 0, 0, 0};
      if (g4 < 3) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          qx[e] = (cq == (uint32_t)(2 * e) ? 0x3F80u : 0u) | (cq == (uint32_t)(2 * e + 1) ? 0x3F800000u : 0u);
      } else {
        qx[0] = 0x3F80u;
      }
      const bf16x8_t qxb = __builtin_bit_cast(bf16x8_t, qx);
      bf16x8_t xf[kNT];
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt) {
        const uint32_t ck = codeS[kt * 16 + l16];
        const uint32_t row = ck == kPadCode ? 8u : ck;
        xf[kt] = *reinterpret_cast<const bf16x8_t*>(smem + kXtOff + (row * 4 + g4) * 16);
      }
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt) {
        S[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[kt], qxb, S[kt], 0, 0, 0);
        WATTN_PIN_MFMA_LDS();
      }
    }

    float mx = S[0][0];
#pragma unroll
    for (int kt = 0; kt < kNT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, S[kt][i]);
    mx = wave_max16x4(mx);
    const float nm = -mx * c2;
    bf16x8_t Pb[4];
    bf16x4_t Pt;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Pb[j][i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(S[2 * j][i], c2, nm));
        Pb[j][4 + i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(S[2 * j + 1][i], c2, nm));
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) Pt[i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(S[8][i], c2, nm));

    const int e = l16 >> 2, qd = l16 & 3;
    auto v_off = [&](int key, int d) { return kTensorBytes + qkv_off(key, d >> 3) + ((d & 4) << 1); };
    floatx4 O[4], L;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const short4_t a4 = lds_tr(smem, v_off(128 + 4 * g4 + e, dbase(t, qd)));
      O[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a4, __builtin_bit_cast(short4_t, Pt),
                                                       floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      WATTN_PIN_MFMA();
    }
    {
      const u32x2 ones2 = u32x2{0x3F803F80u, 0x3F803F80u};
      L = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, ones2),
                                                    __builtin_bit_cast(short4_t, Pt), floatx4{0.f, 0.f, 0.f, 0.f},
                                                    0, 0, 0);
      WATTN_PIN_MFMA();
    }
    u32x4 vf[2][4];
    auto vread = [&](int j, int buf) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const short4_t lo = lds_tr(smem, v_off(32 * j + 4 * g4 + e, dbase(t, qd)));
        const short4_t hi = lds_tr(smem, v_off(32 * j + 16 + 4 * g4 + e, dbase(t, qd)));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
        vf[buf][t] = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
      }
    };
    vread(0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j + 1 < 4) vread(j + 1, (j + 1) & 1);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        O[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vf[j & 1][t]), Pb[j], O[t], 0, 0, 0);
        WATTN_PIN_MFMA_LDS();
      }
      L = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ones), Pb[j], L, 0, 0, 0);
      WATTN_PIN_MFMA_LDS();
    }

    const int32_t tq = tokS[qt * 16 + l16];
    if (tq >= 0) {
      const float inv = __builtin_amdgcn_rcpf(L[0]);
      uint16_t* out = o + (size_t)tq * RS + hoff;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x2 w = u32x2{pack_bf16x2(O[t][0] * inv, O[t][1] * inv), pack_bf16x2(O[t][2] * inv, O[t][3] * inv)};
        *reinterpret_cast<u32x2*>(out + dbase(t, g4)) = w;
      }
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

hipError_t launch_bf16(const swin3d_wattn_plan* pl, const void* q, const void* k, const void* v, void* o,
                       hipStream_t s) {
  AttnParams p;
  const swin3d_wattn_desc_t& d = pl->desc;
  p.X[0] = d.D;
  p.X[1] = d.H;
  p.X[2] = d.W;
  for (int a = 0; a < 3; ++a) {
    p.P[a] = pl->padded[a];
    p.shift[a] = d.shift[a];
    p.win[a] = d.window[a];
    p.nwin[a] = pl->nwin[a];
    for (int j = 0; j < 3; ++j) p.special[a][j] = pl->special[a][j];
  }
  p.heads = d.heads;
  p.n_items = (int32_t)pl->n_items;
  p.c2 = pl->c2;
  p.beta01 = (uint32_t)pl->beta_bf16[0] | ((uint32_t)pl->beta_bf16[1] << 16);
  p.beta2 = pl->beta_bf16[2];
  p.pad = pl->pad_bf16;
  for (int n = 0; n < kN; ++n) p.slot[n] = pl->slot[n];
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  uint16_t* oo = static_cast<uint16_t*>(o);
  void* args[] = {&qq, &kk, &vv, &oo, &p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&wattn_bf16_item), dim3((unsigned)pl->n_items),
                         dim3(kThreads), args, 0, s);
}

}  // namespace

int swin3d_wattn_launch(const swin3d_wattn_plan* p, const void* q, const void* k, const void* v, void* o,
                        void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (p->kernel == 1) {
    e = launch_bf16(p, q, k, v, o, s);
  } else if (p->desc.head_dim == 32) {
    e = launch_f32<32>(p, q, k, v, o, s);
  } else {
    e = launch_f32<64>(p, q, k, v, o, s);
  }
  return e == hipSuccess ? SWIN3D_WATTN_OK : SWIN3D_WATTN_ELAUNCH;
}
