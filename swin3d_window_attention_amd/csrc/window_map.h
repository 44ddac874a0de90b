// Device-side window geometry shared by the FP32, split-bf16, K/V-streaming
// and whole-window kernels: the index map from a window slot to its grid
// token (pad, cyclic shift, 3D partition; Flash-Aurora README, "Kernel
// fusion for backbone memory traffic") and the shift-region code of the
// slot ("Window attention kernels": tokens of different regions of a
// shifted window do not attend to each other), plus small helpers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.h"
#include "plan.h"

namespace wmap {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef __bf16 bf16x4_t __attribute__((__vector_size__(8)));
typedef short short4_t __attribute__((__vector_size__(8)));
typedef float floatx4 __attribute__((__vector_size__(16)));
typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
typedef uint32_t u32x2 __attribute__((__vector_size__(8)));

constexpr uint32_t kPadSlot = 8;  // region code of a padding slot

using fastdiv::FastDiv;
using fastdiv::fdiv;
using fastdiv::make_fastdiv;

// Grid, padding, shift and window of a plan, and the windows that hold a
// region cut or padding along each axis (-1 = none)
struct Geom {
  int32_t X[3], P[3], shift[3], win[3], nwin[3];
  int32_t special[3][3];
  int32_t padwin[3][2];         // windows that hold padding along each axis (-1 = none)
  int32_t N;                    // slots per window
  FastDiv div_b, div_d, div_h;  // by windows per batch element, per depth slab, per row
  FastDiv div_hw, div_w;        // by window slots per depth step, per row
};

inline Geom make_geom(const swin3d_wattn_plan* pl) {
  Geom g;
  const swin3d_wattn_desc_t& d = pl->desc;
  g.X[0] = d.D;
  g.X[1] = d.H;
  g.X[2] = d.W;
  for (int a = 0; a < 3; ++a) {
    g.P[a] = pl->padded[a];
    g.shift[a] = d.shift[a];
    g.win[a] = d.window[a];
    g.nwin[a] = pl->nwin[a];
    for (int j = 0; j < 3; ++j) g.special[a][j] = pl->special[a][j];
    for (int j = 0; j < 2; ++j) g.padwin[a][j] = pl->padwin[a][j];
  }
  g.N = pl->N;
  g.div_b = make_fastdiv((uint32_t)(pl->nwin[0] * pl->nwin[1] * pl->nwin[2]));
  g.div_d = make_fastdiv((uint32_t)(pl->nwin[1] * pl->nwin[2]));
  g.div_h = make_fastdiv((uint32_t)pl->nwin[2]);
  g.div_hw = make_fastdiv((uint32_t)(d.window[1] * d.window[2]));
  g.div_w = make_fastdiv((uint32_t)d.window[2]);
  return g;
}

struct WinPos {
  int b, k[3];
  uint32_t tok0;  // token of slot 0 when the window has no cut and no padding
  bool masked;    // the window has a region cut or padding along some axis
  bool padded;    // the window holds padding slots
};

// Window w (batch folded in) -> (b, kd, kh, kw)
__device__ __forceinline__ WinPos decode_window(const Geom& g, uint32_t w) {
  WinPos it;
  const uint32_t per_d = (uint32_t)(g.nwin[1] * g.nwin[2]);
  it.b = (int)fdiv(w, g.div_b);
  w -= (uint32_t)it.b * per_d * (uint32_t)g.nwin[0];
  it.k[0] = (int)fdiv(w, g.div_d);
  w -= (uint32_t)it.k[0] * per_d;
  it.k[1] = (int)fdiv(w, g.div_h);
  it.k[2] = (int)(w - (uint32_t)it.k[1] * (uint32_t)g.nwin[2]);
  bool m = false;
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int j = 0; j < 3; ++j) m |= g.special[a][j] == it.k[a];
  it.masked = m;
  bool pd = false;
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int j = 0; j < 2; ++j) pd |= g.padwin[a][j] == it.k[a];
  it.padded = pd;
  // without a cut or padding no slot wraps or falls outside the grid: slot
  // (od, oh, ow) is token tok0 + (od H + oh) W + ow
  it.tok0 = (((uint32_t)it.b * (uint32_t)g.X[0] + (uint32_t)(it.k[0] * g.win[0] + g.shift[0])) * (uint32_t)g.X[1] +
             (uint32_t)(it.k[1] * g.win[1] + g.shift[1])) * (uint32_t)g.X[2] +
            (uint32_t)(it.k[2] * g.win[2] + g.shift[2]);
  return it;
}

// Slot n = (od, oh, ow) of the window (row-major) -> its token and region
// code: one bit per axis, set where the shifted position lies in [P - s, P)
// (empty when s = 0), or kPadSlot for padding. Padding, and any slot n >= N
// (the tail of a last chunk or query block), gets a real stand-in token, the
// nearest one on the grid (each coordinate clamped to X - 1), so that loads
// need no condition: a padding key gets a zero weight and a padding query is
// never written. kTail = false: the caller's n is always below N.
template <bool kTail = true>
__device__ __forceinline__ void map_slot(const Geom& g, const WinPos& it, uint32_t n, int32_t& tok, uint32_t& code) {
  const bool beyond = kTail && n >= (uint32_t)g.N;
  n = beyond ? 0u : n;
  int o[3];
  o[0] = (int)fdiv(n, g.div_hw);
  const uint32_t r = n - (uint32_t)o[0] * (uint32_t)(g.win[1] * g.win[2]);
  o[1] = (int)fdiv(r, g.div_w);
  o[2] = (int)(r - (uint32_t)o[1] * (uint32_t)g.win[2]);
  int gc[3];
  uint32_t c = 0;
  bool valid = !beyond;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    const int pa = it.k[a] * g.win[a] + o[a];
    int ga = pa + g.shift[a];
    ga = ga >= g.P[a] ? ga - g.P[a] : ga;
    valid = valid && ga < g.X[a];
    gc[a] = min(ga, g.X[a] - 1);
    c |= (g.shift[a] > 0 && pa >= g.P[a] - g.shift[a]) ? (1u << a) : 0u;
  }
  tok = ((it.b * g.X[0] + gc[0]) * g.X[1] + gc[1]) * g.X[2] + gc[2];
  code = valid ? c : kPadSlot;
}

// map_slot for a window without a cut or padding (it.masked false) and n < N:
// every slot is a real token of region 0
__device__ __forceinline__ int32_t map_slot_plain(const Geom& g, const WinPos& it, uint32_t n) {
  const uint32_t o0 = fdiv(n, g.div_hw);
  const uint32_t r = n - o0 * (uint32_t)(g.win[1] * g.win[2]);
  const uint32_t o1 = fdiv(r, g.div_w);
  const uint32_t o2 = r - o1 * (uint32_t)g.win[2];
  return (int32_t)(it.tok0 + (o0 * (uint32_t)g.X[1] + o1) * (uint32_t)g.X[2] + o2);
}

// element offset of token t's row in a tensor of token stride s (< 2^31):
// one 32 x 32 -> 64-bit multiply
__device__ __forceinline__ size_t row_at(int32_t t, uint32_t s) { return (uint64_t)(uint32_t)t * s; }

// Q, K, V rows are read once: non-temporal 16-byte loads
template <typename T>
__device__ __forceinline__ u32x4 ldg16(const T* ptr) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr));
}

// ds_read_b64_tr_b16: within each 16-lane group, input lane 4e + q points
// at 4 dims of key e and output lane m receives key e of dim 4 (m / 4) + m % 4
__device__ __forceinline__ short4_t lds_tr(const uint8_t* smem, int byte_off) {
  typedef short4_t __attribute__((address_space(3))) * lds_ptr;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(smem + byte_off));
}

// max / sum over the four lanes l16 + 16 g4: lane ^ 16 by a swizzle within
// each half-wave (bit mode: and 0x1F, xor 0x10), lane ^ 32 by a permute whose
// byte address x32 = 4 (lane ^ 32) the caller computes once
__device__ __forceinline__ float wave_max16x4(float x, int x32) {
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(x32, __builtin_bit_cast(int, x))));
  return x;
}
__device__ __forceinline__ float wave_sum16x4(float x, int x32) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
  x += __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(x32, __builtin_bit_cast(int, x)));
  return x;
}

}  // namespace wmap
