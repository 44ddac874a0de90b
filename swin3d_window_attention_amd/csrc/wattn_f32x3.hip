// Swin3D shifted-window attention kernel, FP32 I/O on the matrix cores, for
// gfx950 (MI355X).
//
// This is the FP32-fidelity precision mode of the path: the Flash-Aurora
// README ("Window attention kernels", "Precision tiers") runs FP32 inputs and
// outputs through reduced-precision tensor-core products with FP32
// accumulation (its TF32_ACC_FP32 mode). gfx950 has no TF32/XF32 matrix
// instruction, and FP32 matrix products run at 1/16 of the bf16 rate, so
// every product here is formed from bf16 splits instead: x = hi + lo with
// hi = bf16(x) and lo = bf16(x - hi) (both round-to-nearest-even), and
//   A B ~= Ah Bh + Al Bh + Ah Bl
// with FP32 accumulation. The dropped Al Bl term and the part of x below lo
// are each about 2^-16 of |x|, so products carry ~16 significant bits: finer
// than TF32's 11, coarser than FP32's 24. The softmax is FP32 throughout.
//
// Structure follows the bf16 kernel: one workgroup of four waves per
// (window, head), head-major launch grid (window, head), integer index map
// for pad / cyclic shift / partition (README, "Kernel fusion for backbone
// memory traffic"), the shifted-window bias and the padding exclusion as an
// extra matrix-core k-step, single K/V tile in LDS ("CuTe DSL window
// attention"), O scattered straight back to grid layout.
//
// LDS: hi and lo bf16 splits of K and of V (four 144 x 64 tiles, 72 KB), so
// two workgroups share a CU. K and V are split once, when they are written
// to LDS; Q is split in registers, P right after the exponential.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"
#include "window_map.h"

namespace {

using namespace wmap;

// Matrix-core ordering (see the bf16 kernel): an MFMA whose accumulator
// input comes from one of the last few MFMAs reads its A/B registers late,
// so consecutive MFMAs use independent accumulators and the order is pinned.
#define X3_PIN_MFMA() __builtin_amdgcn_sched_barrier(0x7F6)
#define X3_PIN_MFMA_LDS() __builtin_amdgcn_sched_barrier(0x676)

constexpr int kN = 144;
constexpr int kNT = 9;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxQT = (kNT + kWaves - 1) / kWaves;
constexpr int kTile = kN * 128;  // one 144 x 64 bf16 tile
// LDS layout (bytes): K hi, K lo, V hi, V lo, key and query mask-feature
// tables (9 codes x 4 lane groups x 16 B each), region code and token of
// each slot
constexpr int kKh = 0;
constexpr int kKl = kTile;
constexpr int kVh = 2 * kTile;
constexpr int kVl = 3 * kTile;
constexpr int kXtOff = 4 * kTile;
constexpr int kQtOff = kXtOff + 9 * 4 * 16;
constexpr int kCodeOff = kQtOff + 9 * 4 * 16;
constexpr int kTokOff = kCodeOff + kN;
constexpr int kSmemBytes = kTokOff + kN * 4;

struct AttnParams {
  Geom g;                       // grid, padding, shift, window
  int64_t sq, sk, sv, so;       // token strides of Q, K, V, O (elements)
  float c2;                     // scale * log2(e)
  uint32_t beta01;              // bf16 bias/scale terms 0 | 1 << 16
  uint32_t beta2;               // bf16 bias/scale term 2
  uint32_t pad;                 // bf16 padding-key offset
};

__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 1) | (((r >> 3) & 1) << 1) | (((r >> 2) & 1) << 2); }
// byte offset of 16-byte chunk c (0..7) of row r in a 128-byte-row bf16 tile
__device__ __forceinline__ int qkv_off(int r, int c) { return r * 128 + ((c ^ swz(r)) << 4); }
// first dim of the 4-dim group q held by output tile t (conflict-free transposed V reads)
__device__ __forceinline__ int dbase(int t, int q) { return (t >> 1) * 32 + q * 8 + 4 * ((q ^ t) & 1); }


// Four fp32 values -> their hi and lo bf16 splits (round to nearest even).
// Written with whole-vector conversions: building the bf16 vectors element by
// element and reading an element back was miscompiled (every element taken
// from element 0) by the ROCm 7.2 compiler.
__device__ __forceinline__ void split4f(floatx4 f, bf16x4_t& hi, bf16x4_t& lo) {
  hi = __builtin_convertvector(f, bf16x4_t);
  lo = __builtin_convertvector(f - __builtin_convertvector(hi, floatx4), bf16x4_t);
}

__device__ __forceinline__ void split4(u32x4 x, u32x2& hi, u32x2& lo) {
  bf16x4_t h, l;
  split4f(__builtin_bit_cast(floatx4, x), h, l);
  hi = __builtin_bit_cast(u32x2, h);
  lo = __builtin_bit_cast(u32x2, l);
}

__device__ __forceinline__ bf16x8_t cat8(bf16x4_t a, bf16x4_t b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void wattn_f32x3_item(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v, float* __restrict__ o,
    const AttnParams p) {
  __shared__ __align__(16) uint8_t smem[kSmemBytes];
  uint8_t* codeS = smem + kCodeOff;
  int32_t* tokS = reinterpret_cast<int32_t*>(smem + kTokOff);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  const int x32 = (lane ^ 32) << 2;  // byte address of lane ^ 32 for ds_bpermute
  const int head = blockIdx.y;
  const WinPos cur = decode_window(p.g, blockIdx.x);
  const size_t hoff = (size_t)head * 64;

  // ---- gather: K and V rows whole (sixteen lanes x 16 B per 256-byte row).
  // The sixteen lanes of a row share its slot map: the lane of chunk j maps
  // the row of the group's load j and writes that row's slot table entry
  // (token, region code) for the mask and the scatter; every lane takes the
  // token of its load j from that lane by a permute, bit 31 flagging a
  // padding slot ----
  constexpr int kChunks = kN * 16;
  constexpr int kPer = kChunks / kThreads;
  static_assert(kChunks % kThreads == 0 && kPer <= 16, "whole chunks per thread, one row per lane");
  // Padding slots load a stand-in token; their K and V rows are replaced by
  // zeros before they reach LDS, so the stand-in's values never reach an
  // output (an Inf or NaN in it stays in its own window).
  u32x4 kr[kPer], vr[kPer];
  uint32_t padk = 0;  // bit j: load j is a padding slot's stand-in
  const int gbase = (lane & ~15) * 4;  // byte address of the row group's first lane
  int32_t mtok = 0;
  if ((tid & 15) < kPer) {
    const int r = (tid >> 4) + (kThreads / 16) * (tid & 15);
    int32_t t;
    uint32_t code;
    map_slot<false>(p.g, cur, (uint32_t)r, t, code);
    tokS[r] = t;
    codeS[r] = (uint8_t)code;
    mtok = code == kPadSlot ? (int32_t)((uint32_t)t | 0x80000000u) : t;
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int c = tid + kThreads * j;
    int32_t t = __builtin_amdgcn_ds_bpermute(gbase + 4 * j, mtok);
    padk |= t < 0 ? 1u << j : 0u;
    t &= 0x7FFFFFFF;
    kr[j] = ldg16(k + (size_t)t * p.sk + hoff + 4 * (c & 15));
    vr[j] = ldg16(v + (size_t)t * p.sv + hoff + 4 * (c & 15));
  }
  // Q straight into the operand layout: lane (g4, query l16) of a tile holds
  // dims [8 g4, 8 g4 + 8) and the same + 32 of its query row
  u32x4 qr[kMaxQT][4];
#pragma unroll
  for (int qi = 0; qi < kMaxQT; ++qi) {
    const int qt = wave + kWaves * qi;
    if (qt < kNT) {
      int32_t t;
      uint32_t unused;
      map_slot<false>(p.g, cur, (uint32_t)(qt * 16 + l16), t, unused);
      const float* base = q + (size_t)t * p.sq + hoff + 8 * g4;
      qr[qi][0] = ldg16(base);
      qr[qi][1] = ldg16(base + 4);
      qr[qi][2] = ldg16(base + 32);
      qr[qi][3] = ldg16(base + 36);
    }
  }
  // ---- K and V into LDS as hi / lo bf16 tiles: fp32 chunk `part` (dims
  // 4 part .. 4 part + 3) is one 8-byte half of bf16 chunk part / 2 ----
  if (cur.padded) {  // wave-uniform
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (padk & (1u << j)) kr[j] = vr[j] = u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int c = tid + kThreads * j;
    const int part = c & 15;
    const int off = qkv_off(c >> 4, part >> 1) + (part & 1) * 8;
    u32x2 h, l;
    split4(kr[j], h, l);
    *reinterpret_cast<u32x2*>(smem + kKh + off) = h;
    *reinterpret_cast<u32x2*>(smem + kKl + off) = l;
    split4(vr[j], h, l);
    *reinterpret_cast<u32x2*>(smem + kVh + off) = h;
    *reinterpret_cast<u32x2*>(smem + kVl + off) = l;
  }
  // ---- mask-feature tables (windows with a cut or padding only), built by
  // the last wave (the slot table was written during the gather) ----
  if (cur.masked && tid >= kThreads - 64) {
    for (int e = tid - (kThreads - 64); e < 72; e += 64) {
      const uint32_t ck = (e < 36 ? e : e - 36) >> 2, part = e & 3;
      u32x4 w = u32x4{0, 0, 0, 0};
      if (e < 36) {
        // key: bias / scale at every region other than its own (three bf16
        // terms, exact to float precision), the padding offset (part 3)
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
#pragma unroll
  for (int qi = 0; qi < kMaxQT; ++qi) {
    const int qt = wave + kWaves * qi;
    if (qt >= kNT) break;
    bf16x8_t qh[2], ql[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x4_t h0, l0, h1, l1;
      split4f(__builtin_bit_cast(floatx4, qr[qi][2 * s]), h0, l0);
      split4f(__builtin_bit_cast(floatx4, qr[qi][2 * s + 1]), h1, l1);
      qh[s] = cat8(h0, h1);
      ql[s] = cat8(l0, l1);
    }

    // ---- S^T = K Q^T: per 32-dim step, three blocks of nine MFMAs (one per
    // key tile): Kh Qh, Kl Qh, Kh Ql ----
    floatx4 S[kNT];
#pragma unroll
    for (int kt = 0; kt < kNT; ++kt) S[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8_t kh[kNT], kl[kNT];
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt) {
        const int off = qkv_off(kt * 16 + l16, 4 * s + g4);
        kh[kt] = *reinterpret_cast<const bf16x8_t*>(smem + kKh + off);
        kl[kt] = *reinterpret_cast<const bf16x8_t*>(smem + kKl + off);
      }
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt) {
        S[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh[kt], qh[s], S[kt], 0, 0, 0);
        X3_PIN_MFMA();
      }
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt) {
        S[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl[kt], qh[s], S[kt], 0, 0, 0);
        X3_PIN_MFMA();
      }
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt) {
        S[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh[kt], ql[s], S[kt], 0, 0, 0);
        X3_PIN_MFMA();
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
        X3_PIN_MFMA_LDS();
      }
    }

    // ---- softmax in FP32 (log2 domain), P split into hi / lo B operands; the
    // row sum adds the FP32 values (it differs from the sum of the splits by
    // less than the dropped lo-lo products) ----
    float mx = S[0][0];
#pragma unroll
    for (int kt = 0; kt < kNT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, S[kt][i]);
    mx = wave_max16x4(mx, x32);
    const float nm = -mx * c2;
    floatx4 P[kNT];
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < kNT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        P[kt][i] = __builtin_amdgcn_exp2f(fmaf(S[kt][i], c2, nm));
        rs += P[kt][i];
      }
    bf16x8_t Ph[4], Pl[4];
    bf16x4_t Pth, Ptl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4_t ah, al, bh, bl;
      split4f(P[2 * j], ah, al);
      split4f(P[2 * j + 1], bh, bl);
      Ph[j] = cat8(ah, bh);
      Pl[j] = cat8(al, bl);
    }
    split4f(P[8], Pth, Ptl);

    const float inv = 1.0f / wave_sum16x4(rs, x32);

    // ---- O^T = V^T P^T: Vh Ph, Vl Ph, Vh Pl ----
    const int e = l16 >> 2, qd = l16 & 3;
    auto v_off = [&](int tile, int key, int d) { return tile + qkv_off(key, d >> 3) + ((d & 4) << 1); };
    floatx4 O[4];
    {
      short4_t ah[4], al[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        ah[t] = lds_tr(smem, v_off(kVh, 128 + 4 * g4 + e, dbase(t, qd)));
        al[t] = lds_tr(smem, v_off(kVl, 128 + 4 * g4 + e, dbase(t, qd)));
      }
      const short4_t pth = __builtin_bit_cast(short4_t, Pth), ptl = __builtin_bit_cast(short4_t, Ptl);
      const floatx4 zero = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        O[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah[t], pth, zero, 0, 0, 0);
        X3_PIN_MFMA();
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        O[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al[t], pth, O[t], 0, 0, 0);
        X3_PIN_MFMA();
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        O[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah[t], ptl, O[t], 0, 0, 0);
        X3_PIN_MFMA();
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 vh[4], vl[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int d = dbase(t, qd);
        const u32x2 a = __builtin_bit_cast(u32x2, lds_tr(smem, v_off(kVh, 32 * j + 4 * g4 + e, d)));
        const u32x2 b = __builtin_bit_cast(u32x2, lds_tr(smem, v_off(kVh, 32 * j + 16 + 4 * g4 + e, d)));
        const u32x2 c = __builtin_bit_cast(u32x2, lds_tr(smem, v_off(kVl, 32 * j + 4 * g4 + e, d)));
        const u32x2 f = __builtin_bit_cast(u32x2, lds_tr(smem, v_off(kVl, 32 * j + 16 + 4 * g4 + e, d)));
        vh[t] = u32x4{a[0], a[1], b[0], b[1]};
        vl[t] = u32x4{c[0], c[1], f[0], f[1]};
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        O[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vh[t]), Ph[j], O[t], 0, 0, 0);
        X3_PIN_MFMA();
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        O[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vl[t]), Ph[j], O[t], 0, 0, 0);
        X3_PIN_MFMA();
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        O[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vh[t]), Pl[j], O[t], 0, 0, 0);
        X3_PIN_MFMA();
      }
    }

    // ---- normalise and scatter: tile t holds dims dbase(t, g4) .. + 3 of query l16 ----
    if (codeS[qt * 16 + l16] != kPadSlot) {
      float* out = o + (size_t)tokS[qt * 16 + l16] * p.so + hoff;
#pragma unroll
      for (int t = 0; t < 4; ++t) *reinterpret_cast<floatx4*>(out + dbase(t, g4)) = O[t] * inv;
    }
  }
}

hipError_t launch(const swin3d_wattn_plan* pl, const void* q, const void* k, const void* v, void* o,
                  const swin3d_wattn_strides_t* st, hipStream_t s) {
  AttnParams p;
  const swin3d_wattn_desc_t& d = pl->desc;
  p.g = make_geom(pl);
  p.sq = st->q;
  p.sk = st->k;
  p.sv = st->v;
  p.so = st->o;
  p.c2 = pl->c2;
  p.beta01 = (uint32_t)pl->beta_bf16[0] | ((uint32_t)pl->beta_bf16[1] << 16);
  p.beta2 = pl->beta_bf16[2];
  p.pad = pl->pad_bf16;
  const float* qq = static_cast<const float*>(q);
  const float* kk = static_cast<const float*>(k);
  const float* vv = static_cast<const float*>(v);
  float* oo = static_cast<float*>(o);
  void* args[] = {&qq, &kk, &vv, &oo, &p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&wattn_f32x3_item),
                         dim3((unsigned)pl->n_windows, (unsigned)d.heads), dim3(kThreads), args, 0, s);
}

}  // namespace

int wattn_launch_f32x3(const swin3d_wattn_plan* p, const void* q, const void* k, const void* v, void* o,
                       const swin3d_wattn_strides_t* stride, void* stream) {
  return (int)launch(p, q, k, v, o, stride, static_cast<hipStream_t>(stream));
}
