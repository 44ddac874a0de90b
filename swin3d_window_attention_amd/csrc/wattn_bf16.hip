// Swin3D shifted-window attention kernel, BF16 I/O on the matrix cores, for gfx950
// (MI355X).
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

#include <type_traits>

#include "fastdiv.h"
#include "plan.h"

namespace {

// ---------------------------------------------------------------------------
// BF16 path: matrix-core kernel for N = 144 tokens per window (window
// (2, 6, 12) or any other with 144 slots) and head_dim 64.
//
// Work: one workgroup of four waves per (window, head) item, launch grid
// (window, head) so that dispatch is head-major: the workgroups in flight
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
constexpr uint32_t kPadSlot = 8;          // region code of a padding slot
// LDS layout (bytes): K tile, V tile, the key and the query mask-feature
// tables (9 codes x 4 lane groups x 16 B each), then the region code and
// the token of each slot
constexpr int kXtOff = 2 * kTensorBytes;
constexpr int kQtOff = kXtOff + 9 * 4 * 16;
constexpr int kCodeOff = kQtOff + 9 * 4 * 16;
constexpr int kTokOff = kCodeOff + kN;
constexpr int kSmemBytes = kTokOff + kN * 4;

using fastdiv::FastDiv;
using fastdiv::fdiv;
using fastdiv::make_fastdiv;

// Division as in fastdiv.h, for the per-lane slot arithmetic, where n < 2^8
// (a slot of the 144-token window) and d <= 2^12, with a fixed shift in full-rate 24-bit
// operations: mul = ceil(2^20 / d) <= 2^20, so n * mul < 2^28, and the error
// term n * (mul * d - 2^20) < 2^8 * 2^12 stays below 2^20: the quotient is
// exact, and it is known to fit 12 bits, so it feeds the next 24-bit product
// unmasked.
constexpr uint32_t kSmallShr = 20;

uint32_t make_small_div(uint32_t d) { return (uint32_t)(((uint64_t(1) << kSmallShr) + d - 1) / d); }

__device__ __forceinline__ uint32_t fdiv_small(uint32_t n, uint32_t mul) { return __umul24(n, mul) >> kSmallShr; }

struct AttnParams {
  int32_t X[3], P[3], shift[3], win[3], nwin[3];
  int32_t special[3][3];
  int32_t padwin[3][2];  // windows that hold padding along each axis (-1 = none)
  FastDiv div_b, div_d, div_h;  // by windows per batch, per depth slab, per row
  uint32_t div_hw, div_w;       // fdiv_small multipliers by wh * ww and by ww
  uint32_t whw;                 // wh * ww
  uint32_t plane;               // H * W tokens
  uint32_t sq, sk, sv, so;      // token strides of Q, K, V, O (elements, < 2^31)
  float c2;
  uint32_t beta01;  // bf16 beta term 0 | term 1 << 16
  uint32_t beta2;   // bf16 beta term 2
  uint32_t pad;     // bf16 padding-key offset
};

__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 1) | (((r >> 3) & 1) << 1) | (((r >> 2) & 1) << 2); }
// byte offset of 16-byte chunk c (0..7) of row r in a 128-byte-row tensor tile
__device__ __forceinline__ int qkv_off(int r, int c) { return r * 128 + ((c ^ swz(r)) << 4); }
// first dim of the 4-dim group q (0..3) held by output tile t (0..3); the
// alternation of the +4 between neighbouring groups makes each transposed
// read touch both 8-byte halves of the 16-byte chunks it spans
__device__ __forceinline__ int dbase(int t, int q) { return (t >> 1) * 32 + q * 8 + 4 * ((q ^ t) & 1); }

// max over the four lanes l16 + 16 g4: lane ^ 16 by a swizzle within each
// half-wave (bit mode: and 0x1F, xor 0x10), lane ^ 32 by a permute whose
// byte address x32 = 4 (lane ^ 32) the caller computes once
__device__ __forceinline__ float wave_max16x4(float x, int x32) {
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(x32, __builtin_bit_cast(int, x))));
  return x;
}

struct WinPos {
  int b, k[3];
  int base[3];    // first padded-grid coordinate of the window, k * w
  uint32_t tokb;  // first token of batch element b
  uint32_t tok0;  // token of slot 0 when the window has no cut and no padding
  bool masked;
  bool padded;    // the window holds padding slots
};

// Window w (batch folded in) -> (b, kd, kh, kw) and whether it needs the
// mask path (a region cut or padding along some axis).
__device__ __forceinline__ WinPos decode_window(const AttnParams& p, uint32_t w) {
  WinPos it;
  const uint32_t per_d = (uint32_t)(p.nwin[1] * p.nwin[2]);
  it.b = (int)fdiv(w, p.div_b);
  w -= (uint32_t)it.b * per_d * (uint32_t)p.nwin[0];
  it.k[0] = (int)fdiv(w, p.div_d);
  w -= (uint32_t)it.k[0] * per_d;
  it.k[1] = (int)fdiv(w, p.div_h);
  it.k[2] = (int)(w - (uint32_t)it.k[1] * (uint32_t)p.nwin[2]);
  for (int a = 0; a < 3; ++a) it.base[a] = it.k[a] * p.win[a];
  it.tokb = (uint32_t)it.b * (uint32_t)p.X[0] * p.plane;
  bool m = false;
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int j = 0; j < 3; ++j) m |= p.special[a][j] == it.k[a];
  it.masked = m;
  bool pd = false;
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int j = 0; j < 2; ++j) pd |= p.padwin[a][j] == it.k[a];
  it.padded = pd;
  // without a cut or padding on any axis no slot wraps or falls outside the
  // grid, so slot (od, oh, ow) is token tok0 + od H W + oh W + ow
  it.tok0 = it.tokb + (uint32_t)(it.base[0] + p.shift[0]) * p.plane +
            (uint32_t)(it.base[1] + p.shift[1]) * (uint32_t)p.X[2] + (uint32_t)(it.base[2] + p.shift[2]);
  return it;
}

// Grid position of slot n = (od, oh, ow) (row-major inside the window, n <
// 2^8) and its region code (one bit per axis: position in the wrapped part
// [P - s, P), empty when s = 0), or kPadSlot for padding. A padding slot
// still gets a real token, the nearest one on the grid (each coordinate
// clamped to X - 1), so that all loads can be unconditional. Per lane this
// is full-rate 24-bit arithmetic except one 32-bit product (g0 * H * W).
// kEdge = false is the shortcut for windows without a cut or padding
// (it.masked false, a wave-uniform condition): every code is 0 there.
template <bool kEdge>
__device__ __forceinline__ void map_slot(const AttnParams& p, const WinPos& it, uint32_t n, int32_t& tok,
                                         uint32_t& code) {
  uint32_t o[3];
  o[0] = fdiv_small(n, p.div_hw);
  const uint32_t r = n - __umul24(o[0], p.whw);
  o[1] = fdiv_small(r, p.div_w);
  o[2] = r - __umul24(o[1], (uint32_t)p.win[2]);
  if (!kEdge) {
    tok = (int32_t)(it.tok0 + o[0] * p.plane + __umul24(o[1], (uint32_t)p.X[2]) + o[2]);
    code = 0;
    return;
  }
  int g[3];
  uint32_t c = 0;
  bool valid = true;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    const int pa = it.base[a] + (int)o[a];
    int ga = pa + p.shift[a];
    ga = ga >= p.P[a] ? ga - p.P[a] : ga;
    valid = valid && ga < p.X[a];
    g[a] = min(ga, p.X[a] - 1);
    c |= pa >= p.P[a] - p.shift[a] ? (1u << a) : 0u;
  }
  tok = (int32_t)(it.tokb + (uint32_t)g[0] * p.plane + __umul24((uint32_t)g[1], (uint32_t)p.X[2]) + (uint32_t)g[2]);
  code = valid ? c : kPadSlot;
}

// element offset of token t's row in a tensor of token stride s (< 2^31):
// added to a per-lane column pointer, one 32 x 32 + 64-bit multiply-add
__device__ __forceinline__ size_t row_off(int32_t t, uint32_t s) { return (uint64_t)(uint32_t)t * s; }

// Q, K and V rows are read exactly once per launch. Where Q, K and V together
// exceed the 256 MB Infinity Cache, a non-temporal load marks each line as
// streaming, so it does not displace useful lines in L2 or that cache
// (measured on MI355X for this gather pattern: 5.9 TB/s with non-temporal
// loads against 5.0 TB/s with ordinary ones). Inputs that fit in the cache
// are read with ordinary loads (kKeep): a launch then finds them there when
// their producer, or the previous launch on the same inputs, left them
// there. Output stores stay ordinary (non-temporal stores were slower).
template <bool kKeep>
__device__ __forceinline__ u32x4 ldg16(const uint16_t* ptr) {
  if constexpr (kKeep)
    return *reinterpret_cast<const u32x4*>(ptr);
  else
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr));
}

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

template <bool kKeep>
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
  const int x32 = (lane ^ 32) << 2;  // byte address of lane ^ 32 for ds_bpermute
  // grid (window, head): x varies fastest, so the workgroups in flight read
  // one head of many neighbouring windows
  const int head = blockIdx.y;
  const WinPos cur = decode_window(p, blockIdx.x);
  const uint32_t hoff = (uint32_t)head * 64;

  // ---- gather first: each thread maps the slots it loads itself, so the
  // loads leave before any table or barrier. K and V rows go to registers
  // (then LDS), the Q operands of this wave's tiles stay in registers.
  // Padding slots read their stand-in token (so every load is unconditional)
  // and their K and V rows are replaced by zeros before they reach LDS: a
  // padding key then gets an exactly zero weight and adds exactly zero
  // whatever the stand-in holds (an Inf or NaN there stays in its own
  // window); a padding query is never written. ----
  constexpr int kChunks = kN * 8;
  constexpr int kPer = (kChunks + kThreads - 1) / kThreads;
  u32x4 kr[kPer], vr[kPer];
  // every load of a thread reads 16-byte chunk tid % 8 (K, V) or lane % 8 (Q)
  // of its row: the same column, tid % 8 = lane % 8
  const uint32_t col = hoff + 8 * (uint32_t)(tid & 7);
  const uint16_t* kcol = k + col;
  const uint16_t* vcol = v + col;
  const uint16_t* qcol = q + col;
  uint16_t* ocol = o + col;  // the output stores write chunk lane % 8 too
  // Q rows of this wave's tiles are read whole: load s of a tile covers its
  // rows 8 s .. 8 s + 7, lane L reading 16-byte chunk L % 8 of row 8 s + L / 8
  u32x4 qr[kMaxQT][2];
  uint32_t padk = 0;  // bit j: load j of this thread is a padding slot's stand-in
  auto gather = [&](auto edge) {
    constexpr bool kEdge = decltype(edge)::value;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int c = tid + kThreads * j;
      if (c < kChunks) {
        int32_t t;
        uint32_t code;
        map_slot<kEdge>(p, cur, (uint32_t)(c >> 3), t, code);
        kr[j] = ldg16<kKeep>(kcol + row_off(t, p.sk));
        vr[j] = ldg16<kKeep>(vcol + row_off(t, p.sv));
        if (kEdge) padk |= code == kPadSlot ? 1u << j : 0u;
      }
    }
#pragma unroll
    for (int qi = 0; qi < kMaxQT; ++qi) {
      const int qt = wave + kWaves * qi;
      if (qt < kNT) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          int32_t t;
          uint32_t unused;
          map_slot<kEdge>(p, cur, (uint32_t)(qt * 16 + 8 * s + (lane >> 3)), t, unused);
          qr[qi][s] = ldg16<kKeep>(qcol + row_off(t, p.sq));
        }
      }
    }
  };
  // one uniform branch: windows without a cut or padding take the shortcut
  if (cur.masked)
    gather(std::true_type{});
  else
    gather(std::false_type{});

  if (cur.padded) {  // wave-uniform
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (padk & (1u << j)) kr[j] = vr[j] = u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int c = tid + kThreads * j;
    if (c < kChunks) {
      *reinterpret_cast<u32x4*>(smem + qkv_off(c >> 3, c & 7)) = kr[j];
      *reinterpret_cast<u32x4*>(smem + kTensorBytes + qkv_off(c >> 3, c & 7)) = vr[j];
    }
  }
  // ---- the slot table (token, region code) for the mask and the scatter ----
  for (int r = tid; r < kN; r += kThreads) {
    int32_t t;
    uint32_t c;
    if (cur.masked)
      map_slot<true>(p, cur, (uint32_t)r, t, c);
    else
      map_slot<false>(p, cur, (uint32_t)r, t, c);
    tokS[r] = t;
    codeS[r] = (uint8_t)c;
  }
  // ---- mask-feature tables (windows with a cut or padding only), built by
  // the wave that has no slots to map ----
  if (cur.masked && tid >= kThreads - 64) {
    for (int e = tid - (kThreads - 64); e < 72; e += 64) {
      const uint32_t ck = (e < 36 ? e : e - 36) >> 2, part = e & 3;
      u32x4 w = u32x4{0, 0, 0, 0};
      if (e < 36) {
        // key: bias / scale at every region other than its own (three bf16
        // terms, parts 0..2), the padding offset in the padding column (part 3)
        const uint32_t beta[3] = {p.beta01 & 0xFFFFu, p.beta01 >> 16, p.beta2 & 0xFFFFu};
        if (ck == kPadSlot) {
          if (part == 3) w[0] = p.pad;
        } else if (part < 3) {
          const uint32_t bt = beta[part];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t lo = (uint32_t)(2 * i) != ck ? bt : 0u;
            const uint32_t hi = (uint32_t)(2 * i + 1) != ck ? bt : 0u;
            w[i] = lo | (hi << 16);
          }
        }
      } else if (part < 3) {
        // query: a one-hot of its region in each of the three slots
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = ((uint32_t)(2 * i) == ck ? 0x3F80u : 0u) | ((uint32_t)(2 * i + 1) == ck ? 0x3F800000u : 0u);
      } else {
        w[0] = 0x3F80u;  // query: 1 in the padding column
      }
      *reinterpret_cast<u32x4*>(smem + kXtOff + e * 16) = w;
    }
  }
  __syncthreads();

  const float c2 = p.c2;
  const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
  for (int qi = 0; qi < kMaxQT; ++qi) {
    const int qt = wave + kWaves * qi;
    if (qt >= kNT) break;
    // B operand of S^T: lane (g4, query l16) needs dims [8 g4, 8 g4 + 8) and
    // the same + 32 of its query row, i.e. chunks g4 and g4 + 4. Move them
    // over from the whole-row layout: lanes with chunk >= 4 first take the
    // second load's value from 4 lanes down (and those with chunk < 4 the
    // first load's from 4 lanes up), so one pull per dword serves both halves
    bf16x8_t qop[2];
    {
      const bool lo = (lane & 7) < 4;
      const int src = 4 * (8 * (l16 & 7) + g4 + 4 * (l16 >> 3));
      u32x4 q0, q1;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t a = qr[qi][0][d], b = qr[qi][1][d];
        const uint32_t b_down = (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0x124, 0xF, 0xF, false);  // lane i - 4
        const uint32_t a_up = (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0x12C, 0xF, 0xF, false);    // lane i + 4
        q0[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(lo ? a : b_down));
        q1[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(lo ? a_up : b));
      }
      qop[0] = __builtin_bit_cast(bf16x8_t, q0);
      qop[1] = __builtin_bit_cast(bf16x8_t, q1);
    }

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
      const bf16x8_t qxb =
          *reinterpret_cast<const bf16x8_t*>(smem + kQtOff + (codeS[qt * 16 + l16] * 4 + g4) * 16);
      bf16x8_t xf[kNT];
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt)
        xf[kt] = *reinterpret_cast<const bf16x8_t*>(smem + kXtOff + (codeS[kt * 16 + l16] * 4 + g4) * 16);
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
    mx = wave_max16x4(mx, x32);
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

    // normalise and pack: with the dbase() order, lane (g4, query l16) holds
    // dims [8 g4, 8 g4 + 8) in tiles t = 0, 1 and the same dims + 32 in t = 2, 3
    const float inv = __builtin_amdgcn_rcpf(L[0]);
    uint32_t w[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      w[t][0] = pack_bf16x2(O[t][0] * inv, O[t][1] * inv);
      w[t][1] = pack_bf16x2(O[t][2] * inv, O[t][3] * inv);
    }
    const bool odd = g4 & 1;
    const u32x4 c0 = odd ? u32x4{w[1][0], w[1][1], w[0][0], w[0][1]} : u32x4{w[0][0], w[0][1], w[1][0], w[1][1]};
    const u32x4 c1 = odd ? u32x4{w[3][0], w[3][1], w[2][0], w[2][1]} : u32x4{w[2][0], w[2][1], w[3][0], w[3][1]};
    // exchange so that each store instruction writes eight whole 128-byte
    // rows: store s, lane L -> row 8 s + L / 8, 16-byte chunk L % 8. Chunk ch < 4
    // of row r is c0 of lane (ch, r); chunk ch >= 4 is c1 of lane (ch - 4, r),
    // first rotated by 8 lanes inside its 16-lane row so that one pull per
    // dword serves both halves
    u32x4 z;
#pragma unroll
    for (int d = 0; d < 4; ++d) z[d] = (uint32_t)__builtin_amdgcn_mov_dpp((int)c1[d], 0x128, 0xF, 0xF, false);
    const int ch = lane & 7, rr = lane >> 3;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bool mine = (l16 >> 3) == s;
      const int src = ch < 4 ? (ch * 16 + 8 * s + rr) : ((ch - 4) * 16 + 8 * (1 - s) + rr);
      u32x4 val;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        val[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(src * 4, (int)(mine ? c0[d] : z[d]));
      const int r = qt * 16 + 8 * s + rr;
      if (codeS[r] != kPadSlot)
        *reinterpret_cast<u32x4*>(ocol + row_off(tokS[r], p.so)) = val;
    }
  }
}

hipError_t launch(const swin3d_wattn_plan* pl, const void* q, const void* k, const void* v, void* o,
                  const swin3d_wattn_strides_t* st, hipStream_t s) {
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
    for (int j = 0; j < 2; ++j) p.padwin[a][j] = pl->padwin[a][j];
  }
  p.div_b = make_fastdiv((uint32_t)(pl->nwin[0] * pl->nwin[1] * pl->nwin[2]));
  p.div_d = make_fastdiv((uint32_t)(pl->nwin[1] * pl->nwin[2]));
  p.div_h = make_fastdiv((uint32_t)pl->nwin[2]);
  p.c2 = pl->c2;
  p.beta01 = (uint32_t)pl->beta_bf16[0] | ((uint32_t)pl->beta_bf16[1] << 16);
  p.beta2 = pl->beta_bf16[2];
  p.pad = pl->pad_bf16;
  p.sq = (uint32_t)st->q;
  p.sk = (uint32_t)st->k;
  p.sv = (uint32_t)st->v;
  p.so = (uint32_t)st->o;
  p.whw = (uint32_t)(d.window[1] * d.window[2]);
  p.plane = (uint32_t)(d.H * d.W);
  p.div_hw = make_small_div(p.whw);
  p.div_w = make_small_div((uint32_t)d.window[2]);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  uint16_t* oo = static_cast<uint16_t*>(o);
  void* args[] = {&qq, &kk, &vv, &oo, &p};
  // ordinary loads where Q, K and V together fit in the 256 MB Infinity Cache
  const bool keep = 3 * pl->elems * pl->elem_bytes <= (int64_t(256) << 20);
  return hipLaunchKernel(keep ? reinterpret_cast<const void*>(&wattn_bf16_item<true>)
                              : reinterpret_cast<const void*>(&wattn_bf16_item<false>),
                         dim3((unsigned)pl->n_windows, (unsigned)d.heads), dim3(kThreads), args, 0, s);
}

}  // namespace

int wattn_launch_bf16(const swin3d_wattn_plan* p, const void* q, const void* k, const void* v, void* o,
                      const swin3d_wattn_strides_t* stride, void* stream) {
  return (int)launch(p, q, k, v, o, stride, static_cast<hipStream_t>(stream));
}
