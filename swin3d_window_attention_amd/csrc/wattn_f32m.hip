// Swin3D shifted-window attention, exact FP32 on the matrix cores, for gfx950
// (MI355X): windows of N = 144 slots, head_dim 32 or 64.
//
// This is the FP32 path of the method at matrix-core speed: both products
// run on v_mfma_f32_16x16x4_f32 (FP32 operands, FP32 accumulation, no
// reduced-precision step anywhere); the shifted-window mask is the FP32
// initial value of the Q K^T accumulators, read from a per-window table of
// query code x key terms, and the softmax and P stay in FP32 on the vector
// ALU. The Flash-Aurora README
// ("Window attention kernels", "CuTe DSL window attention") keeps the whole
// window's K and V in one shared-memory tile; so does this kernel.
//
// Work: one workgroup of four waves per (window, head), head-major launch
// grid (window, head); the nine 16-query tiles of a window are dealt to the
// waves with a rotation by workgroup, so the wave that takes three tiles
// does not always sit on the same SIMD. Index map for pad / cyclic shift /
// partition and the scatter back to grid layout as in the other kernels
// ("Kernel fusion for backbone memory traffic").
//
// Layouts (16x16x4 FP32 MFMA: lane l holds A[l % 16][l / 16] and
// B[l / 16][l % 16]; the result D[4 (l / 16) + i][l % 16], i = 0..3):
//  S^T = K Q^T: A = 16 keys x 4 dims of K, B = 4 dims x 16 queries of Q^T.
//    The contraction order over dims is free, so k-step s of lane group kk
//    takes dim kk DH/4 + s: a lane's K and Q values are contiguous and come
//    four at a time (16-byte loads). K is row-major in LDS, 16-byte chunks
//    XOR-swizzled by row, so these reads are conflict-free.
//  O^T = V^T P^T: the S^T accumulator gives lane (g4, query) keys
//    16 kt + 4 g4 + i, which is the B operand of k-step (kt, i) with
//    key(kk) = 16 kt + 4 kk + i; P never leaves registers. The A operand
//    (dims x those keys) is read from V stored transposed in LDS (rows of
//    144 keys, padded to 148 floats so the 16 rows of a read hit distinct
//    banks): lane (kk, dim m) gets keys 16 kt + 4 kk .. + 3, the operands of
//    four consecutive k-steps, in one 16-byte read.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "plan.h"
#include "window_map.h"

namespace {

using namespace wmap;

// Matrix-core ordering: consecutive MFMAs use independent accumulators (an
// MFMA whose accumulator input comes from one of the last few MFMAs reads
// its A/B registers late). The scheduling barrier pins the MFMA order; the
// empty volatile asm statements around each MFMA (on its A operand before,
// on its accumulator after) also stop instruction selection from moving a
// pure MFMA, which the barrier cannot undo. They emit no instruction.
#define FM_PIN_MFMA() __builtin_amdgcn_sched_barrier(0x7F6)
#define FM_BEFORE(a) asm volatile("" : "+v"(a))
#define FM_AFTER(c) asm volatile("" : "+v"(c))

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// window of N <= 16 NT slots, NT key / query tiles of 16 (slots N .. 16 NT - 1 are padding)
template <int DH, int NT>
struct Lds {
  static constexpr int kN = 16 * NT;
  static constexpr int kVtPitch = kN + 4;            // floats per transposed-V row (16 rows hit distinct banks)
  static constexpr int kK = 0;                       // K, row-major, kN x DH floats
  static constexpr int kVt = kN * DH * 4;            // V^T, DH x kVtPitch floats
  static constexpr int kCode = kVt + DH * kVtPitch * 4;
  static constexpr int kTok = kCode + kN;            // 4-byte aligned: kN is a multiple of 16
  static constexpr int kBias = kTok + kN * 4;        // mask terms, 9 query codes x kN keys floats
  static constexpr int kBytes = kBias + 9 * kN * 4;
};

struct AttnParams {
  Geom g;                       // grid, padding, shift, window
  int64_t sq, sk, sv, so;       // token strides of Q, K, V, O (elements)
  float c2;                     // scale * log2(e)
  float bias_s;                 // cross-region bias / scale (may be -inf)
};

// byte offset of 16-byte chunk c of K row r (DH / 4 chunks per row, XOR-swizzled by row)
template <int DH>
__device__ __forceinline__ int k_off(int r, int c) {
  return r * (DH * 4) + ((c ^ (r & (DH / 4 - 1))) << 4);
}

template <int DH, int NT, bool kTail>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Lds<DH, NT>::kBytes > 80 * 1024 ? 1 : 2))) void wattn_f32m_item(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v, float* __restrict__ o,
    const AttnParams p) {
  using L = Lds<DH, NT>;
  constexpr int kN = L::kN;                   // slots, N of them real (N > 16 (NT - 1))
  constexpr int kNT = NT;                     // key / query tiles of 16
  constexpr int kVtPitch = L::kVtPitch;
  constexpr int kCh = DH / 4;                 // 16-byte chunks per row
  constexpr int kQC = DH / 16;                // 16-byte chunks of a lane's dims (= k-step groups of 4)
  constexpr int kT = DH / 16;                 // 16-dim output tiles
  constexpr int kAccP = kT >= 4 ? 1 : 2;      // P V accumulator sets (independent neighbours)
  constexpr int kChunks = kN * kCh;
  constexpr int kPer = (kChunks + kThreads - 1) / kThreads;
  constexpr int kMaxQT = (kNT + kWaves - 1) / kWaves;
  __shared__ __align__(16) uint8_t smem[L::kBytes];
  uint8_t* codeS = smem + L::kCode;
  int32_t* tokS = reinterpret_cast<int32_t*>(smem + L::kTok);
  float* vt = reinterpret_cast<float*>(smem + L::kVt);
  float* biasS = reinterpret_cast<float*>(smem + L::kBias);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  const int x32 = (lane ^ 32) << 2;  // byte address of lane ^ 32 for ds_bpermute
  const int head = blockIdx.y;
  const WinPos cur = decode_window(p.g, blockIdx.x);
  const size_t hoff = (size_t)head * DH;
  // query tiles of this wave: (wave - rot) mod 4 + 4 i; the rotation moves
  // the three-tile share from wave to wave across workgroups
  const int rot = (int)((blockIdx.x + blockIdx.y) & 3u);
  const int first = (wave - rot) & 3;

  // ---- gather: K and V rows whole (kCh lanes x 16 B per row), each thread
  // mapping the slots it loads; Q straight into the B-operand layout ----
  // Padding slots load a stand-in token; their K and V rows are replaced by
  // zeros before they reach LDS, so the stand-in's values never reach an
  // output (an Inf or NaN in it stays in its own window).
  // The kCh lanes that load one row share its slot map: lane (chunk) ch maps
  // the row of load ch and writes the slot table entry (token, region code)
  // of that row and that key's column of the mask table (the term added to
  // Q K^T for each of the nine query codes); every lane takes the token of
  // its load j from lane j of its group by a permute, bit 31 flagging a
  // padding slot.
  static_assert((kCh == 8 || kCh == 16) && kPer <= kCh, "row groups inside one wave, one row per lane");
  u32x4 kr[kPer], vr[kPer];
  uint32_t padk = 0;  // bit j: load j is a padding slot's stand-in
  const int gbase = (lane & ~(kCh - 1)) * 4;  // byte address of the group's first lane
  int32_t mtok = 0;
  {
    const int r = tid / kCh + (kThreads / kCh) * (tid % kCh);
    if (tid % kCh < kPer && r < kN) {
      int32_t t;
      uint32_t code;
      map_slot<kTail>(p.g, cur, (uint32_t)r, t, code);
      tokS[r] = t;
      codeS[r] = (uint8_t)code;
      mtok = code == kPadSlot ? (int32_t)((uint32_t)t | 0x80000000u) : t;
      // mask term of key r for a query of code c, in the units of Q K^T: the
      // cross-region bias / scale where both are real and their regions
      // differ, -inf for a padding key, 0 otherwise (a padding query, never
      // written, takes no bias; in a window without a cut or padding every
      // slot has code 0, so the row its queries read is all zeros)
#pragma unroll
      for (uint32_t c = 0; c <= kPadSlot; ++c)
        biasS[c * kN + r] = code == kPadSlot ? -INFINITY : (c != kPadSlot && code != c ? p.bias_s : 0.f);
    }
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int c = tid + kThreads * j;
    if (c < kChunks) {
      int32_t t = __builtin_amdgcn_ds_bpermute(gbase + 4 * j, mtok);
      padk |= t < 0 ? 1u << j : 0u;
      t &= 0x7FFFFFFF;
      kr[j] = ldg16(k + (size_t)t * p.sk + hoff + 4 * (c % kCh));
      vr[j] = ldg16(v + (size_t)t * p.sv + hoff + 4 * (c % kCh));
    }
  }
  // lane (kk = g4, query l16) of a tile holds dims kk DH/4 .. + DH/4 - 1. Up to
  // ten tiles, every tile's Q is loaded here; beyond, the first tile's here and
  // each later one during the tile before it (the compiler may keep that tile
  // loop rolled, so no register array in it is indexed by the tile)
  constexpr int kPre = kNT > 10 ? 1 : kMaxQT;
  auto load_q = [&](int qt, floatx4 (&dst)[kQC]) {
    int32_t t;
    uint32_t unused;
    map_slot<kTail>(p.g, cur, (uint32_t)(qt * 16 + l16), t, unused);
    const float* base = q + (size_t)t * p.sq + hoff + g4 * (DH / 4);
#pragma unroll
    for (int c = 0; c < kQC; ++c) dst[c] = __builtin_bit_cast(floatx4, ldg16(base + 4 * c));
  };
  floatx4 qf[kPre][kQC];
#pragma unroll
  for (int qi = 0; qi < kPre; ++qi)
    if (first + kWaves * qi < kNT) load_q(first + kWaves * qi, qf[qi]);
  // ---- K row-major (swizzled), V transposed into LDS ----
  if (cur.padded || kTail) {  // wave-uniform: padding slots, or slots past N in the last tile
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (padk & (1u << j)) kr[j] = vr[j] = u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int c = tid + kThreads * j;
    if (c < kChunks) {
      const int r = c / kCh, ch = c % kCh;
      *reinterpret_cast<u32x4*>(smem + L::kK + k_off<DH>(r, ch)) = kr[j];
      const floatx4 x = __builtin_bit_cast(floatx4, vr[j]);
#pragma unroll
      for (int e = 0; e < 4; ++e) vt[(4 * ch + e) * kVtPitch + r] = x[e];
    }
  }
  // (the slot table for the mask and the scatter was written during the gather)
  __syncthreads();

  const float c2 = p.c2;
  floatx4 qn[kQC];  // beyond ten tiles: the next tile's Q, loaded during this one
#pragma unroll
  for (int qi = 0; qi < kMaxQT; ++qi) {
    const int qt = first + kWaves * qi;
    if (qt >= kNT) break;
    constexpr bool kRolling = kNT > 10;
    const int qs = kRolling ? 0 : qi;  // this tile's Q operands: qf[qs]
    if (kRolling && qi > 0) {
#pragma unroll
      for (int c = 0; c < kQC; ++c) qf[0][c] = qn[c];
    }
    if (kRolling && qt + kWaves < kNT) load_q(qt + kWaves, qn);


    // ---- S^T = K Q^T: k-step s = 4 c + e of lane group kk is dim kk DH/4 + s ----
    // with fewer than four key tiles, k-step s accumulates into set s % kAccS,
    // so that no MFMA takes its accumulator from one of the three before it.
    // The first set starts from the mask terms of this lane's query code and
    // keys (the cross-region bias / scale where the two regions differ, -inf
    // for a padding key, else 0), so the products accumulate onto the bias in
    // the units of Q K^T.
    const uint32_t qc = codeS[qt * 16 + l16];
    constexpr int kAccS = kNT >= 4 ? 1 : kNT == 1 ? 4 : 2;
    floatx4 S2[kAccS][kNT];
    {
      const float* brow = biasS + qc * kN + 4 * g4;
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt) S2[0][kt] = *reinterpret_cast<const floatx4*>(brow + 16 * kt);
    }
#pragma unroll
    for (int a = 1; a < kAccS; ++a)
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt) S2[a][kt] = floatx4{0.f, 0.f, 0.f, 0.f};
    // beyond ten key tiles the K operands are read a group of tiles at a time
    // (4 or 7, a divisor of NT: the MFMAs of a group alternate between at least
    // four independent accumulators)
    constexpr int kG = kNT <= 10 ? kNT : kNT % 4 == 0 ? 4 : kNT / 2;
    static_assert(kNT % kG == 0 && (kG >= 4 || kG == kNT), "whole groups of at least four tiles");
#pragma unroll
    for (int c = 0; c < kQC; ++c)
#pragma unroll
      for (int g0 = 0; g0 < kNT; g0 += kG) {
        floatx4 kf[kG];
#pragma unroll
        for (int u = 0; u < kG; ++u)
          if (g0 + u < kNT)
            kf[u] = *reinterpret_cast<const floatx4*>(smem + L::kK + k_off<DH>((g0 + u) * 16 + l16, g4 * kQC + c));
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int u = 0; u < kG; ++u)
            if (g0 + u < kNT) {
              floatx4& acc = S2[(4 * c + e) % kAccS][g0 + u];
              float a = kf[u][e];
              FM_BEFORE(a);
              acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, qf[qs][c][e], acc, 0, 0, 0);
              FM_AFTER(acc);
              FM_PIN_MFMA();
            }
      }
    floatx4 S[kNT];
#pragma unroll
    for (int kt = 0; kt < kNT; ++kt) {
      S[kt] = S2[0][kt];
#pragma unroll
      for (int a = 1; a < kAccS; ++a) S[kt] += S2[a][kt];
    }

    // ---- softmax: the row max is subtracted before scaling, so the largest
    // weights see no rounding of a large scaled logit:
    // p = 2^((s - max) scale log2(e)) ----
    float mx = S[0][0];
#pragma unroll
    for (int kt = 0; kt < kNT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, S[kt][i]);
    mx = wave_max16x4(mx, x32);
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < kNT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        S[kt][i] = __builtin_amdgcn_exp2f((S[kt][i] - mx) * c2);  // P, FP32
        rs += S[kt][i];
      }
    const float inv = 1.0f / wave_sum16x4(rs, x32);

    // ---- O^T = V^T P^T: k-step (kt, i) covers keys 16 kt + 4 kk + i ----
    floatx4 O[kAccP][kT];
#pragma unroll
    for (int a = 0; a < kAccP; ++a)
#pragma unroll
      for (int t = 0; t < kT; ++t) O[a][t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < kNT; ++kt) {
      floatx4 va[kT];
#pragma unroll
      for (int t = 0; t < kT; ++t)
        va[t] = *reinterpret_cast<const floatx4*>(vt + (16 * t + l16) * kVtPitch + 16 * kt + 4 * g4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < kT; ++t) {
          float a = va[t][i];
          FM_BEFORE(a);
          O[i % kAccP][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, S[kt][i], O[i % kAccP][t], 0, 0, 0);
          FM_AFTER(O[i % kAccP][t]);
          FM_PIN_MFMA();
        }
    }

    // ---- normalise and scatter: tile t holds dims 16 t + 4 g4 .. + 3 of query l16 ----
    if (qc != kPadSlot) {
      float* out = o + (size_t)tokS[qt * 16 + l16] * p.so + hoff + 4 * g4;
#pragma unroll
      for (int t = 0; t < kT; ++t) {
        const floatx4 r = kAccP == 1 ? O[0][t] : O[0][t] + O[kAccP - 1][t];
        *reinterpret_cast<floatx4*>(out + 16 * t) = r * inv;
      }
    }
  }
}

template <int DH, int NT>
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
  p.bias_s = std::isinf(d.cross_region_bias) ? -INFINITY
                                             : (float)((double)d.cross_region_bias / (double)d.scale);
  const float* qq = static_cast<const float*>(q);
  const float* kk = static_cast<const float*>(k);
  const float* vv = static_cast<const float*>(v);
  float* oo = static_cast<float*>(o);
  void* args[] = {&qq, &kk, &vv, &oo, &p};
  const void* fn = pl->N < 16 * NT ? reinterpret_cast<const void*>(&wattn_f32m_item<DH, NT, true>)
                                    : reinterpret_cast<const void*>(&wattn_f32m_item<DH, NT, false>);
  return hipLaunchKernel(fn,
                         dim3((unsigned)pl->n_windows, (unsigned)d.heads), dim3(kThreads), args, 0, s);
}

}  // namespace

int wattn_launch_f32m(const swin3d_wattn_plan* p, const void* q, const void* k, const void* v, void* o,
                      const swin3d_wattn_strides_t* stride, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the plan admits N <= 256 and head_dim 32 or 64: NT = ceil(N / 16) tiles of 16 slots, above 10
  // rounded up to 12, 14 or 16 (the extra slots are padding)
  const int nt = (p->N + 15) / 16;
  const bool d32 = p->desc.head_dim == 32;
  hipError_t e;
#define F32M_CASE(n) \
  case n:            \
    e = d32 ? launch<32, n>(p, q, k, v, o, stride, s) : launch<64, n>(p, q, k, v, o, stride, s); \
    break;
  switch (nt <= 10 ? nt : nt <= 12 ? 12 : nt <= 14 ? 14 : 16) {
    F32M_CASE(1) F32M_CASE(2) F32M_CASE(3) F32M_CASE(4) F32M_CASE(5) F32M_CASE(6) F32M_CASE(7)
    F32M_CASE(8) F32M_CASE(9) F32M_CASE(10) F32M_CASE(12) F32M_CASE(14) F32M_CASE(16)
    default: e = hipErrorInvalidValue;
  }
#undef F32M_CASE
  return (int)e;
}
