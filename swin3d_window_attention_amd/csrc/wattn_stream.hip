// Swin3D shifted-window attention for any window size and head_dim 32, 64
// or 128, BF16 I/O, for gfx950 (MI355X): two kernels that share the index
// map, the mask tables and the MFMA layouts.
//
// The Flash-Aurora README ("CuTe DSL window attention") keeps K and V of a
// whole window in one shared-memory tile when it fits and otherwise falls
// back to a multi-stage variant that streams K/V through double-buffered
// shared memory. The N = 144, head_dim 64 production shape has its own
// single-tile kernel (four workgroups per CU). Here, wattn_window_item keeps
// the whole window for N x head_dim = 18432 (144 x 128, 288 x 64: two
// workgroups per CU), and wattn_stream_item streams every other window.
//
// wattn_stream_item:
// Work: one workgroup per (window, head, block of query slots), QT = 2 tiles
// of 16 queries per wave (each K and V operand read from LDS serves both);
// K and V of the window pass
// through LDS in chunks of key slots,
// double-buffered: while the waves work on chunk c, each thread holds its
// part of chunk c + 1 in registers and writes it to the other buffer
// afterwards (one barrier per chunk). Two block shapes: four waves and
// 64-key chunks, or, where the window size is a multiple of 48 but not of
// 64 (144, 288, ...), three waves and 48-key chunks, so that no key slot
// past the window is processed (nor a query slot, where N is a multiple of
// the query block; e.g. N = 432). Softmax is online in FP32 (log2 domain):
// a running reference max m per query that moves only when a chunk's max
// exceeds it by more than kLazy in the exponent (O and the row sums then
// rescaled by 2^((m_old - m_new) c2)), row sums of the bf16 P from the
// matrix core.
//
// The index map, the stand-in token for padding slots, the shifted-window
// bias and the padding exclusion as an extra matrix-core k-step, and the
// MFMA layouts (S^T = K Q^T, O^T = V^T P^T with transposing LDS reads) are
// those of the single-tile bf16 kernel. Slots beyond N in the last chunk or
// query block are padding as well.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "plan.h"
#include "window_map.h"

namespace {

using namespace wmap;

// Matrix-core ordering: consecutive MFMAs use independent accumulators (an
// MFMA whose accumulator input comes from one of the last few MFMAs reads
// its A/B registers late) and the order is pinned.
#define ST_PIN_MFMA() __builtin_amdgcn_sched_barrier(0x7F6)
// Instruction selection may still move a pure MFMA (one with a zero
// accumulator in particular) away from its place, which the scheduling
// barrier cannot undo. An empty volatile asm on the A operand before and on
// the accumulator after each MFMA fixes the order: volatile asm statements
// keep their source order, and each MFMA sits between two of them. They emit
// no instruction.
#define ST_BEFORE(a) asm volatile("" : "+v"(a))
#define ST_AFTER(c) asm volatile("" : "+v"(c))
// The same, but LDS instructions stay in place too: used where the source
// issues LDS reads a fixed distance ahead of the MFMAs that consume them.
#define ST_PIN_MFMA_LDS() __builtin_amdgcn_sched_barrier(0x676)

// online softmax: largest exponent (log2) a P value may reach before the
// reference max of its row moves
constexpr float kLazy = 8.0f;

// key slot -> (token, region code) of kRing chunks, refilled four chunks at a time
constexpr int kRing = 8;

template <int DH, int KC>
struct Lds {
  static constexpr int kRow = DH * 2;                // bytes per bf16 row
  static constexpr int kTile = KC * kRow;            // one chunk of K (or V)
  static constexpr int kBuf = 2 * kTile;             // K and V of one chunk
  static constexpr int kXt = 2 * kBuf;               // key feature table
  static constexpr int kQt = kXt + 9 * 4 * 16;       // query feature table
  static constexpr int kTok = kQt + 9 * 4 * 16;      // token of each key slot of the ring's chunks
  static constexpr int kCode = kTok + kRing * KC * 4;  // region code of the same slots
  static constexpr int kBytes = kCode + kRing * KC;
};

struct StreamParams {
  Geom g;          // grid, padding, shift, window
  int32_t nqb;     // query blocks per window
  int32_t nchunk;  // key chunks per window
  int32_t n_windows;
  FastDiv div_qb;  // by query blocks per window
  uint32_t sq, sk, sv, so;  // token strides of Q, K, V, O (elements, < 2^31)
  float c2;
  uint32_t beta01, beta2, pad;
  // K and V token stride in bytes where both are addressed by a 32-bit byte
  // offset from the head's column (equal strides, at most 2^24 tokens, every
  // offset below 2^32); 0: 64-bit addresses
  uint32_t kv2;
};

__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 1) | (((r >> 3) & 1) << 1) | (((r >> 2) & 1) << 2); }
// The row swizzle within the DH / 8 chunks of a row. LDS serves 256 bytes a
// cycle, so what matters is the 16-byte unit within a 256-byte line: rows
// r mod (256 / 2 DH) pick the part of the line, the swizzled chunk the unit
// within it. The swizzle takes the remaining low row bits (3 at DH = 64, 4 at
// 128, 2 at 32), so that one chunk of 16 consecutive rows (a K operand read)
// covers all 16 units, and four consecutive keys at four dim groups (a
// transposing V read) take each unit at most twice, in its two 8-byte halves.
template <int DH>
__device__ __forceinline__ int swzd(int r) {
  if constexpr (DH == 128)
    return swz(r) | ((r & 1) << 3);
  else if constexpr (DH == 64)
    return swz(r);
  else
    return (r >> 2) & 3;
}
// byte offset of 16-byte chunk c of row r
template <int DH>
__device__ __forceinline__ int row_off(int r, int c) { return r * (DH * 2) + ((c ^ swzd<DH>(r)) << 4); }
// byte offset of the 8-byte piece of V row `key` that holds dims d .. d + 3 (d a multiple of 4)
template <int DH>
__device__ __forceinline__ int v_off(int key, int d) {
  return key * (DH * 2) + (((d >> 3) ^ swzd<DH>(key)) << 4) + ((d & 4) << 1);
}
__device__ __forceinline__ int dbase(int t, int q) { return (t >> 1) * 32 + q * 8 + 4 * ((q ^ t) & 1); }

template <int DH, int WAVES, int KC, int QT, bool kPad, bool kOff32>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(DH <= 64 ? 3 : 2))) void wattn_stream_item(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ k,
                                                               const uint16_t* __restrict__ v,
                                                               uint16_t* __restrict__ o, const StreamParams p) {
  using L = Lds<DH, KC>;
  constexpr int kThreads = 64 * WAVES;
  constexpr int kQB = 16 * WAVES * QT;                 // query slots per workgroup (QT tiles per wave)
  constexpr int kKC = KC;                              // key slots per chunk
  constexpr int kKT = KC / 16;                         // key tiles per chunk
  constexpr int kJ = KC / 32;                          // whole 32-key steps of P V
  constexpr bool kTail = KC % 32 != 0;                 // plus one 16-key step
  constexpr int kS = DH / 32;                          // 32-dim k-steps of Q K^T
  constexpr int kT = DH / 16;                          // 16-dim output tiles
  constexpr int kCh = DH / 8;                          // 16-byte chunks per row
  constexpr int kLoads = kKC * kCh / kThreads;         // 16-byte loads per thread per tensor and chunk
  static_assert(kKC * kCh % kThreads == 0, "whole loads per thread");
  static_assert(KC % 16 == 0 && KC <= 64 && kThreads >= 72, "chunk and table sizes");
  __shared__ __align__(16) uint8_t smem[L::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  const int head = blockIdx.y;
  // XCD-aware order: workgroup x runs on XCD x % 8, so x = 8 (w_hi nqb + qb) + w_lo
  // gives window 8 w_hi + w_lo all its query blocks on one XCD, one after the
  // other, where they share that XCD's L2 copy of the window's K and V
  const uint32_t xk = blockIdx.x >> 3;
  const uint32_t w_hi = fdiv(xk, p.div_qb);
  const int qb = (int)(xk - w_hi * (uint32_t)p.nqb);
  const uint32_t wq = 8 * w_hi + (blockIdx.x & 7);
  if (wq >= (uint32_t)p.n_windows) return;  // grid padded to a multiple of 8 windows
  const WinPos cur = decode_window(p.g, wq);
  const size_t hoff = (size_t)head * DH;

  // ---- this wave's QT tiles of 16 queries (tile wave QT + u of the block):
  // Q operands (lane (g4, query l16): dims 32 s + 8 g4 .. + 7), region code,
  // token ----
  int32_t qtok[QT];
  uint32_t qcode[QT];
  bf16x8_t qop[QT][kS];
  bool any_real = false;
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    const int qslot = qb * kQB + (wave * QT + u) * 16 + l16;
    map_slot(p.g, cur, (uint32_t)qslot, qtok[u], qcode[u]);
    any_real |= qcode[u] != kPadSlot;
  }
  // a block whose query slots are all padding writes nothing: it ends here,
  // before loading anything (kPad: the grid needs padding; only windows that
  // hold padding can have such blocks, a wave-uniform test)
  if (kPad && cur.padded) {
    if (!__syncthreads_or(any_real)) return;
  }
  // a wave whose query tiles hold padding or slots past N only (the last
  // block of a window whose size is not a multiple of the block, or a block
  // that runs into padding) loads no Q and forms no scores and no products;
  // it still loads its share of every chunk and meets the barriers
  const bool wave_real = __any(any_real);
  if (wave_real) {
#pragma unroll
    for (int u = 0; u < QT; ++u)
#pragma unroll
      for (int s = 0; s < kS; ++s)
        qop[u][s] = __builtin_bit_cast(bf16x8_t, ldg16(q + row_at(qtok[u], p.sq) + hoff + 32 * s + 8 * g4));
  }

  // ---- chunk loader: thread tid moves 16-byte pieces tid + kThreads i of K and V
  // (key row tid / kCh + i kThreads / kCh, chunk tid % kCh). Chunk 0 maps its own
  // slots; every later chunk reads its key tokens from a ring in LDS (entry
  // c % kRing for chunk c) that all threads fill four chunks at a time, one
  // slot each, four chunks ahead: the slot map costs every wave one
  // evaluation per four chunks ----
  static_assert(kThreads == 4 * kKC, "one ring slot per thread and refill");
  u32x4 kr[kLoads], vr[kLoads];
  int32_t* tok_ring = reinterpret_cast<int32_t*>(smem + L::kTok);
  uint8_t* code_ring = smem + L::kCode;
  static_assert(kThreads % kCh == 0, "one chunk column per thread");
  const int my_row = tid / kCh, my_ch = tid % kCh;
  const uint16_t* kcol = k + hoff + 8 * my_ch;
  const uint16_t* vcol = v + hoff + 8 * my_ch;
  const uint8_t* khead = reinterpret_cast<const uint8_t*>(k + hoff);  // workgroup-uniform bases
  const uint8_t* vhead = reinterpret_cast<const uint8_t*>(v + hoff);
  // Padding slots (and slots past N) load a stand-in, token 0; their K and V
  // rows are replaced by zeros before they reach LDS, so the stand-in's values
  // never reach an output (an Inf or NaN in it stays in its own window). Ring
  // entries carry that flag in bit 31 (tokens are below 2^31).
  uint32_t padk = 0;  // bit i: load i of the chunk in flight is a padding slot's stand-in
  auto fetch = [&](int c) {
    padk = 0;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int r = my_row + (kThreads / kCh) * i;
      int32_t t;
      bool pad;
      if (c == 0) {
        uint32_t code;
        map_slot(p.g, cur, (uint32_t)r, t, code);
        pad = code == kPadSlot;
      } else {
        t = tok_ring[(c % kRing) * kKC + r];
        pad = t < 0;
      }
      padk |= pad ? 1u << i : 0u;
      // every padding slot of the chunk reads token 0 instead of its own
      // stand-in: the same few lines, served from the caches
      t = pad ? 0 : t;
      // ordinary (not non-temporal) loads: the query blocks of a window read
      // the same K and V rows one after another on one XCD, from its L2
      if constexpr (kOff32) {  // one 24-bit multiply-add per row, the same offset into K and V
        const uint32_t off = __umul24((uint32_t)t, p.kv2) + 16u * (uint32_t)my_ch;
        kr[i] = *reinterpret_cast<const u32x4*>(khead + off);
        vr[i] = *reinterpret_cast<const u32x4*>(vhead + off);
      } else {
        kr[i] = *reinterpret_cast<const u32x4*>(kcol + row_at(t, p.sk));
        vr[i] = *reinterpret_cast<const u32x4*>(vcol + row_at(t, p.sv));
      }
    }
  };
  // zero the stand-in rows of chunk c (wave-uniform: only chunks of a window
  // with a cut or padding, or running past N, hold padding slots)
  auto clear_pad = [&](int c) {
    if (cur.padded || (c + 1) * kKC > p.g.N) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i)
        if (padk & (1u << i)) kr[i] = vr[i] = u32x4{0, 0, 0, 0};
    }
  };
  // tokens and region codes of chunks c0 .. c0 + 3 (those that exist) into the ring
  auto fill_ring = [&](int c0) {
    const int c = c0 + tid / kKC, r = tid % kKC;
    if (c < p.nchunk) {
      int32_t t;
      uint32_t code;
      map_slot(p.g, cur, (uint32_t)(c * kKC + r), t, code);
      tok_ring[(c % kRing) * kKC + r] = code == kPadSlot ? (int32_t)((uint32_t)t | 0x80000000u) : t;
      code_ring[(c % kRing) * kKC + r] = (uint8_t)code;
    }
  };

  // mask-feature tables: also unmasked windows use them when the last chunk
  // runs past N
  if (tid < 72) {
    const int e = tid;
    const uint32_t ck = (e < 36 ? e : e - 36) >> 2, part = e & 3;
    u32x4 w = u32x4{0, 0, 0, 0};
    if (e < 36) {
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
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = ((uint32_t)(2 * i) == ck ? 0x3F80u : 0u) | ((uint32_t)(2 * i + 1) == ck ? 0x3F800000u : 0u);
    } else {
      w[0] = 0x3F80u;
    }
    *reinterpret_cast<u32x4*>(smem + L::kXt + e * 16) = w;
  }
  // chunk 0 into buffer 0
  fetch(0);
  clear_pad(0);
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = my_row + (kThreads / kCh) * i;
    *reinterpret_cast<u32x4*>(smem + row_off<DH>(r, my_ch)) = kr[i];
    *reinterpret_cast<u32x4*>(smem + L::kTile + row_off<DH>(r, my_ch)) = vr[i];
  }
  fill_ring(0);  // chunks 0 .. 3
  __syncthreads();

  const float c2 = p.c2;
  float m[QT];
  floatx4 O[QT][kT];
  floatx4 Ls[QT];  // row sums of P on the matrix core (ones x P^T), rescaled with O
  bf16x8_t qxb[QT];
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    m[u] = -INFINITY;
    Ls[u] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kT; ++t) O[u][t] = floatx4{0.f, 0.f, 0.f, 0.f};
    qxb[u] = *reinterpret_cast<const bf16x8_t*>(smem + L::kQt + (qcode[u] * 4 + g4) * 16);
  }
  const int e = l16 >> 2, qd = l16 & 3;
  const int x32 = (lane ^ 32) << 2;
  // bf16 1.0 x 8 / x 4, the A operand of the row-sum products: one register
  // set for the whole loop (the empty asm before each use pins the order)
  u32x4 ones8 = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  u32x2 ones4 = u32x2{0x3F803F80u, 0x3F803F80u};

  // ---- a chunk of padding keys only (possible in a window that holds
  // padding) adds nothing: their weights are exactly zero, so it is neither
  // loaded nor computed. The test reads the chunk's codes in the ring, which
  // were written at least one barrier earlier (workgroup-uniform: every wave
  // reads the same codes) ----
  auto all_pad = [&](int c) -> bool {
    const uint8_t* cp = code_ring + (c % kRing) * kKC;
    bool kp = true;
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt) kp = kp && cp[kt * 16 + l16] == kPadSlot;
    return __all(kp);
  };
  bool skip = kPad && cur.padded && all_pad(0);
  // the chunk loop runs two chunks per trip, so that the buffer of each is
  // a compile-time constant (LDS offsets as immediates)
  auto step = [&](int c, auto buf_) {
      constexpr int buf = decltype(buf_)::value;  // = c & 1
      const uint8_t* kb = smem + buf * L::kBuf;
      const uint8_t* vb = kb + L::kTile;
      const uint8_t* cb = code_ring + (c % kRing) * kKC;
      const bool more = c + 1 < p.nchunk;
      const bool skip_next = kPad && cur.padded && more && all_pad(c + 1);
      if (more && !skip_next) fetch(c + 1);  // next chunk in flight during this chunk's math
      // chunks c + 4 .. c + 7 into the ring entries of chunks c - 4 .. c - 1,
      // whose last readers (the loads of chunk c - 1, the mask step of chunk
      // c - 1, the padding test of chunk c) finished before the previous barrier
      if (c % 4 == 0 && c + 4 < p.nchunk) fill_ring(c + 4);

      if (!skip && wave_real) {
        // ---- S^T = K Q^T for this chunk's key tiles, each K operand read once
        // for the wave's QT query tiles. Consecutive MFMAs take independent
        // accumulators: with fewer than four per k-step, even and odd k-steps
        // accumulate separately, so that no MFMA takes its accumulator from one
        // of the three before it ----
        constexpr int kAcc = kKT * QT >= 4 ? 1 : 2;
        // the wave's priority is raised while it issues matrix-core work, so
        // that of the waves of a SIMD the one with products ready goes first
        // and the others' vector work fills in behind it
        __builtin_amdgcn_s_setprio(1);
        floatx4 S2[kAcc][QT][kKT];
  #pragma unroll
        for (int a = 0; a < kAcc; ++a)
  #pragma unroll
          for (int u = 0; u < QT; ++u)
  #pragma unroll
            for (int kt = 0; kt < kKT; ++kt) S2[a][u][kt] = floatx4{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
        for (int s = 0; s < kS; ++s) {
          bf16x8_t kf[kKT];
  #pragma unroll
          for (int kt = 0; kt < kKT; ++kt)
            kf[kt] = *reinterpret_cast<const bf16x8_t*>(kb + row_off<DH>(kt * 16 + l16, 4 * s + g4));
  #pragma unroll
          for (int kt = 0; kt < kKT; ++kt)
  #pragma unroll
            for (int u = 0; u < QT; ++u) {
              ST_BEFORE(kf[kt]);
              S2[s % kAcc][u][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kt], qop[u][s], S2[s % kAcc][u][kt], 0, 0, 0);
              ST_AFTER(S2[s % kAcc][u][kt]);
              ST_PIN_MFMA();
            }
        }
        // mask k-step: the window has a cut or padding, or this chunk runs past N
        if (cur.masked || (c + 1) * kKC > p.g.N) {
          bf16x8_t xf[kKT];
  #pragma unroll
          for (int kt = 0; kt < kKT; ++kt)
            xf[kt] = *reinterpret_cast<const bf16x8_t*>(smem + L::kXt + (cb[kt * 16 + l16] * 4 + g4) * 16);
  #pragma unroll
          for (int kt = 0; kt < kKT; ++kt)
  #pragma unroll
            for (int u = 0; u < QT; ++u) {
              ST_BEFORE(xf[kt]);
              S2[kS % kAcc][u][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[kt], qxb[u], S2[kS % kAcc][u][kt], 0, 0, 0);
              ST_AFTER(S2[kS % kAcc][u][kt]);
              ST_PIN_MFMA();
            }
        }

        __builtin_amdgcn_s_setprio(0);
        // ---- online softmax. The chunk maxima of all QT tiles first, then their
        // lane exchanges side by side (each waits on the LDS crossbar once for
        // all tiles), then the exponentials ----
        bf16x8_t Pb[QT][kJ > 0 ? kJ : 1];
        bf16x4_t Pt[QT];
        floatx4 S[QT][kKT];
        float mc[QT];
  #pragma unroll
        for (int u = 0; u < QT; ++u) {
  #pragma unroll
          for (int kt = 0; kt < kKT; ++kt) S[u][kt] = kAcc == 1 ? S2[0][u][kt] : S2[0][u][kt] + S2[kAcc - 1][u][kt];
          // the chunk max, taken from the reference m on (the growth test below
          // compares with m anyway); NaN-propagating maxima need no quieting of
          // their inputs, which saves an instruction per operand the compiler
          // cannot prove canonical
          mc[u] = m[u];
  #pragma unroll
          for (int kt = 0; kt < kKT; ++kt)
  #pragma unroll
            for (int i = 0; i < 4; ++i) mc[u] = __builtin_elementwise_maximum(mc[u], S[u][kt][i]);
        }
        int xs[QT];
  #pragma unroll
        for (int u = 0; u < QT; ++u) xs[u] = __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, mc[u]), 0x401F);
  #pragma unroll
        for (int u = 0; u < QT; ++u) mc[u] = __builtin_elementwise_maximum(mc[u], __builtin_bit_cast(float, xs[u]));
  #pragma unroll
        for (int u = 0; u < QT; ++u) xs[u] = __builtin_amdgcn_ds_bpermute(x32, __builtin_bit_cast(int, mc[u]));
  #pragma unroll
        for (int u = 0; u < QT; ++u) {
          const float mc_w = __builtin_elementwise_maximum(mc[u], __builtin_bit_cast(float, xs[u]));
          // the reference max of a row moves only when the chunk's max exceeds it
          // by more than kLazy in the exponent (always on the first chunk, where
          // m = -inf), so P <= 2^kLazy and most chunks rescale nothing; softmax
          // does not depend on the reference
          const bool grow = (mc_w - m[u]) * c2 > kLazy;
          const float m_new = grow ? mc_w : m[u];
          const float nm = -m_new * c2;
          floatx4 P[kKT];
  #pragma unroll
          for (int kt = 0; kt < kKT; ++kt)
  #pragma unroll
            for (int i = 0; i < 4; ++i) P[kt][i] = __builtin_amdgcn_exp2f(fmaf(S[u][kt][i], c2, nm));
          if (__any(grow)) {  // wave-uniform
            const float alpha = grow ? __builtin_amdgcn_exp2f((m[u] - m_new) * c2) : 1.0f;  // 0 on the first chunk
            Ls[u][0] *= alpha;
  #pragma unroll
            for (int t = 0; t < kT; ++t) O[u][t] *= alpha;
          }
          m[u] = m_new;
  #pragma unroll
          for (int j = 0; j < kJ; ++j)
            Pb[u][j] = __builtin_shufflevector(__builtin_convertvector(P[2 * j], bf16x4_t),
                                               __builtin_convertvector(P[2 * j + 1], bf16x4_t), 0, 1, 2, 3, 4, 5, 6, 7);
          Pt[u] = __builtin_convertvector(P[kKT - 1], bf16x4_t);  // 16-key step (kTail)
        }

        __builtin_amdgcn_s_setprio(1);
        // ---- O^T += V^T P^T over the chunk's 32-key steps, each V operand read
        // once for the wave's QT query tiles ----
  #pragma unroll
        for (int j = 0; j < kJ; ++j) {
          u32x4 vf[kT];
  #pragma unroll
          for (int t = 0; t < kT; ++t) {
            const int d = dbase(t, qd);
            const int lo_off = v_off<DH>(32 * j + 4 * g4 + e, d);
            const int hi_off = v_off<DH>(32 * j + 16 + 4 * g4 + e, d);
            const u32x2 a = __builtin_bit_cast(u32x2, lds_tr(vb, lo_off));
            const u32x2 b = __builtin_bit_cast(u32x2, lds_tr(vb, hi_off));
            vf[t] = u32x4{a[0], a[1], b[0], b[1]};
          }
  #pragma unroll
          for (int t = 0; t < kT; ++t)
  #pragma unroll
            for (int u = 0; u < QT; ++u) {
              O[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vf[t]), Pb[u][j], O[u][t], 0, 0, 0);
              ST_PIN_MFMA();
            }
  #pragma unroll
          for (int u = 0; u < QT; ++u) {
            ST_BEFORE(ones8);
            Ls[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ones8), Pb[u][j], Ls[u], 0, 0, 0);
            ST_AFTER(Ls[u]);
            ST_PIN_MFMA();
          }
        }
        if (kTail) {  // keys 32 kJ .. 32 kJ + 15: v_mfma_f32_16x16x16_bf16
          short4_t vt[kT];
  #pragma unroll
          for (int t = 0; t < kT; ++t) {
            const int d = dbase(t, qd);
            const int key = 32 * kJ + 4 * g4 + e;
            vt[t] = lds_tr(vb, v_off<DH>(key, d));
          }
  #pragma unroll
          for (int t = 0; t < kT; ++t)
  #pragma unroll
            for (int u = 0; u < QT; ++u) {
              O[u][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[t], __builtin_bit_cast(short4_t, Pt[u]), O[u][t], 0, 0, 0);
              ST_PIN_MFMA();
            }
  #pragma unroll
          for (int u = 0; u < QT; ++u) {
            ST_BEFORE(ones4);
            Ls[u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, ones4), __builtin_bit_cast(short4_t, Pt[u]), Ls[u], 0, 0, 0);
            ST_AFTER(Ls[u]);
            ST_PIN_MFMA();
          }
        }
        __builtin_amdgcn_s_setprio(0);
      }

      // ---- next chunk into the other buffer (everyone finished chunk c - 1,
      // the last reader of that buffer, at the previous barrier) ----
      if (more && !skip_next) {
        uint8_t* nb = smem + (buf ^ 1) * L::kBuf;
        clear_pad(c + 1);
  #pragma unroll
        for (int i = 0; i < kLoads; ++i) {
          const int r = my_row + (kThreads / kCh) * i;
          *reinterpret_cast<u32x4*>(nb + row_off<DH>(r, my_ch)) = kr[i];
          *reinterpret_cast<u32x4*>(nb + L::kTile + row_off<DH>(r, my_ch)) = vr[i];
        }
      }
      __syncthreads();
      skip = skip_next;
  };
  for (int c = 0; c < p.nchunk; c += 2) {
    step(c, std::integral_constant<int, 0>{});
    if (c + 1 < p.nchunk) step(c + 1, std::integral_constant<int, 1>{});
  }

  // ---- normalise and scatter (queries of the window only): tiles 2 m and
  // 2 m + 1 hold the two 8-byte halves of the 16-byte chunk at dims
  // 32 m + 8 g4 (tile 2 m first for even g4, second for odd), one store each.
  // (Staging the rows through LDS for whole-row stores measured slower
  // here: the extra round trip sits at the end of every workgroup.) ----
  const bool odd = g4 & 1;
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    if (qcode[u] != kPadSlot) {
      const float inv = 1.0f / Ls[u][0];
      uint16_t* out = o + row_at(qtok[u], p.so) + hoff;
#pragma unroll
      for (int m2 = 0; m2 < kT / 2; ++m2) {
        const u32x2 a = __builtin_bit_cast(u32x2, __builtin_convertvector(O[u][2 * m2] * inv, bf16x4_t));
        const u32x2 b = __builtin_bit_cast(u32x2, __builtin_convertvector(O[u][2 * m2 + 1] * inv, bf16x4_t));
        const u32x4 w = odd ? u32x4{b[0], b[1], a[0], a[1]} : u32x4{a[0], a[1], b[0], b[1]};
        *reinterpret_cast<u32x4*>(out + 32 * m2 + 8 * g4) = w;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Whole-window variant for the shapes whose K and V together fill half of
// the LDS: N x head_dim = 18432 (144 x 128, 288 x 64), 72 KB of K and V plus
// the tables, two workgroups per CU. This is the single-tile case of the
// README's CuTe kernel on a 160 KB LDS: the window's K and V are staged once,
// four waves loop over its query tiles (tile wave + 4 i), and each tile's
// softmax takes one pass over all N keys, so nothing is rescaled and no
// query block re-reads K and V. Index map, stand-in tokens, mask k-step,
// operand layouts and the output stores are the streaming kernel's.
// ---------------------------------------------------------------------------
template <int DH, int NT>
struct WinLds {
  static constexpr int kTensor = 16 * NT * DH * 2;  // K (or V) of the whole window
  static constexpr int kXt = 2 * kTensor;           // key then query feature tables, 72 x 16 B
  static constexpr int kCode = kXt + 72 * 16;       // region code of each slot
  static constexpr int kBytes = kCode + 16 * NT;
};

template <int DH, int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void wattn_window_item(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, const StreamParams p) {
  using L = WinLds<DH, NT>;
  constexpr int kThreads = 256;
  constexpr int kWaves = 4;
  constexpr int kN = 16 * NT;                          // slots of the window (= N)
  constexpr int kS = DH / 32;                          // 32-dim k-steps of Q K^T
  constexpr int kT = DH / 16;                          // 16-dim output tiles
  constexpr int kCh = DH / 8;                          // 16-byte chunks per row
  constexpr int kPer = (kN * kCh + kThreads - 1) / kThreads;  // 16-byte loads per thread and tensor
  constexpr int kMaxQT = (NT + kWaves - 1) / kWaves;   // query tiles per wave (at most)
  constexpr int kJ = kN / 32;                          // whole 32-key steps of P V
  constexpr bool kTail = kN % 32 != 0;                 // plus one 16-key step
  __shared__ __align__(16) uint8_t smem[L::kBytes];
  uint8_t* codeS = smem + L::kCode;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  // grid (window, head), x fastest: the workgroups in flight read one head of
  // many neighbouring windows
  const int head = blockIdx.y;
  const WinPos cur = decode_window(p.g, blockIdx.x);
  const size_t hoff = (size_t)head * DH;

  // ---- gather: K and V rows to registers (then LDS), the Q operands of this
  // wave's tiles to registers; every load leaves before the first barrier ----
  u32x4 kr[kPer], vr[kPer];
  int32_t qtok[kMaxQT];
  uint32_t qcode[kMaxQT];
  bf16x8_t qop[kMaxQT][kS];
  // slot -> token: the full map in windows with a cut or padding, the plain
  // one elsewhere (a wave-uniform branch)
  // load j of thread tid: chunk tid % kCh of row tid / kCh + j kThreads / kCh
  static_assert(kThreads % kCh == 0, "one chunk column per thread");
  const int my_row = tid / kCh, my_ch = tid % kCh;
  const uint16_t* kcol = k + hoff + 8 * my_ch;
  const uint16_t* vcol = v + hoff + 8 * my_ch;
  uint32_t padk = 0;  // bit j: load j of this thread is a padding slot's stand-in
  // The kCh lanes that load one row share its slot map: lane (chunk) c maps
  // the rows of loads c, c + kCh, ... (and, in windows with a cut or padding,
  // writes their region codes for the mask step); every lane takes the token
  // of its load j from lane j mod kCh of its group by a permute, bit 31
  // flagging a padding slot.
  static_assert(kCh == 8 || kCh == 16, "row groups inside one wave");
  constexpr int kMap = (kPer + kCh - 1) / kCh;
  const int gbase = (lane & ~(kCh - 1)) * 4;  // byte address of the group's first lane
  auto gather = [&](auto edge) {
    constexpr bool kEdge = decltype(edge)::value;
    int32_t mtok[kMap];
#pragma unroll
    for (int m = 0; m < kMap; ++m) {
      const int j = my_ch + kCh * m;
      const int r = my_row + (kThreads / kCh) * j;
      mtok[m] = 0;
      if (j < kPer && r < kN) {
        if (kEdge) {
          int32_t t;
          uint32_t code;
          map_slot(p.g, cur, (uint32_t)r, t, code);
          codeS[r] = (uint8_t)code;
          mtok[m] = code == kPadSlot ? (int32_t)((uint32_t)t | 0x80000000u) : t;
        } else {
          mtok[m] = map_slot_plain(p.g, cur, (uint32_t)r);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int r = my_row + (kThreads / kCh) * j;
      if (r < kN) {
        int32_t t = __builtin_amdgcn_ds_bpermute(gbase + 4 * (j % kCh), mtok[j / kCh]);
        if (kEdge) {
          padk |= t < 0 ? 1u << j : 0u;
          t &= 0x7FFFFFFF;
        }
        kr[j] = ldg16(kcol + row_at(t, p.sk));
        vr[j] = ldg16(vcol + row_at(t, p.sv));
      }
    }
#pragma unroll
    for (int i = 0; i < kMaxQT; ++i) {
      const int qt = wave + kWaves * i;
      qcode[i] = kPadSlot;
      if (qt < NT) {
        if (kEdge) {
          map_slot(p.g, cur, (uint32_t)(qt * 16 + l16), qtok[i], qcode[i]);
        } else {
          qtok[i] = map_slot_plain(p.g, cur, (uint32_t)(qt * 16 + l16));
          qcode[i] = 0;
        }
#pragma unroll
        for (int s = 0; s < kS; ++s)
          qop[i][s] = __builtin_bit_cast(bf16x8_t, ldg16(q + row_at(qtok[i], p.sq) + hoff + 32 * s + 8 * g4));
      }
    }
  };
  if (cur.masked)
    gather(std::true_type{});
  else
    gather(std::false_type{});
  // padding slots: zero K and V rows in LDS, so the stand-in's values never
  // reach an output (an Inf or NaN in it stays in its own window)
  if (cur.padded) {
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (padk & (1u << j)) kr[j] = vr[j] = u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int r = my_row + (kThreads / kCh) * j;
    if (r < kN) {
      *reinterpret_cast<u32x4*>(smem + row_off<DH>(r, my_ch)) = kr[j];
      *reinterpret_cast<u32x4*>(smem + L::kTensor + row_off<DH>(r, my_ch)) = vr[j];
    }
  }
  // mask-feature tables: windows with a cut or padding only (their region
  // codes were written during the gather)
  if (cur.masked) {
    if (tid < 72) {
      const int e = tid;
      const uint32_t ck = (e < 36 ? e : e - 36) >> 2, part = e & 3;
      u32x4 w = u32x4{0, 0, 0, 0};
      if (e < 36) {
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
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = ((uint32_t)(2 * i) == ck ? 0x3F80u : 0u) | ((uint32_t)(2 * i + 1) == ck ? 0x3F800000u : 0u);
      } else {
        w[0] = 0x3F80u;
      }
      *reinterpret_cast<u32x4*>(smem + L::kXt + e * 16) = w;
    }
  }
  __syncthreads();

  const float c2 = p.c2;
  const int x32 = (lane ^ 32) << 2;
  const uint8_t* vb = smem + L::kTensor;
  const int e = l16 >> 2, qd = l16 & 3;
  const bool odd = g4 & 1;
  // bf16 1.0 x 8 / x 4, the A operand of the row-sum products: one register
  // set for all tiles (the empty asm before each use pins the order)
  u32x4 ones8 = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  u32x2 ones4 = u32x2{0x3F803F80u, 0x3F803F80u};
  // region codes of this lane's key slots kt 16 + l16 (windows with a cut or
  // padding), four bits each, eight to a register: the mask k-step finds
  // each key's feature without a dependent LDS read
  constexpr int kCW = (NT + 7) / 8;
  uint32_t kcodes[kCW];
#pragma unroll
  for (int w = 0; w < kCW; ++w) kcodes[w] = 0;
  if (cur.masked) {
#pragma unroll
    for (int kt = 0; kt < NT; ++kt) kcodes[kt / 8] |= (uint32_t)codeS[kt * 16 + l16] << (4 * (kt % 8));
  }
  auto tiles = [&](auto mask_) {
    constexpr bool kMask = decltype(mask_)::value;
#pragma unroll
    for (int i = 0; i < kMaxQT; ++i) {
      const int qt = wave + kWaves * i;
      if (qt >= NT) break;

      // ---- S^T = K Q^T over all key tiles; K operands read kAhead MFMAs ahead.
      // k-step s of key tile kt is MFMA s NT + kt, so an accumulator's
      // successive MFMAs lie NT >= 4 apart ----
      floatx4 S[NT];
#pragma unroll
      for (int kt = 0; kt < NT; ++kt) S[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
      {
        // one stream of MFMAs: the Q K^T k-steps (k-step idx / NT of key tile
        // idx % NT), then in windows with a cut or padding the mask k-step of
        // every key tile; A operands (K, or the key's mask feature located by
        // its code) read kAhead MFMAs ahead
        constexpr int kSteps = kS * NT;
        constexpr int kAll = kSteps + (kMask ? NT : 0);
        constexpr int kAhead = 8;
        const bf16x8_t qxb =
            kMask ? *reinterpret_cast<const bf16x8_t*>(smem + L::kXt + (36 + qcode[i] * 4 + g4) * 16) : bf16x8_t{};
        bf16x8_t kf[kAll];
        auto kread = [&](int idx) {
          if (idx < kSteps) {
            const int s = idx / NT, kt = idx % NT;
            kf[idx] = *reinterpret_cast<const bf16x8_t*>(smem + row_off<DH>(kt * 16 + l16, 4 * s + g4));
          } else {
            const int kt = idx - kSteps;
            const uint32_t code = (kcodes[kt / 8] >> (4 * (kt % 8))) & 15u;
            kf[idx] = *reinterpret_cast<const bf16x8_t*>(smem + L::kXt + (code * 4 + g4) * 16);
          }
        };
#pragma unroll
        for (int idx = 0; idx < kAhead; ++idx) kread(idx);
#pragma unroll
        for (int idx = 0; idx < kAll; ++idx) {
          const int kt = idx < kSteps ? idx % NT : idx - kSteps;
          ST_BEFORE(kf[idx]);
          S[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[idx], idx < kSteps ? qop[i][idx / NT] : qxb, S[kt], 0, 0, 0);
          ST_AFTER(S[kt]);
          ST_PIN_MFMA_LDS();
          if (idx + kAhead < kAll) kread(idx + kAhead);
        }
      }

      // ---- softmax in FP32 (log2 domain), P to bf16 in the B-operand layout;
      // NaN-propagating maxima need no quieting of their inputs ----
      float mx = S[0][0];
#pragma unroll
      for (int kt = 0; kt < NT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = __builtin_elementwise_maximum(mx, S[kt][r]);
      mx = __builtin_elementwise_maximum(
          mx, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, mx), 0x401F)));
      mx = __builtin_elementwise_maximum(
          mx, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(x32, __builtin_bit_cast(int, mx))));
      const float nm = -mx * c2;
      bf16x8_t Pb[kJ > 0 ? kJ : 1];
      bf16x4_t Pt, prev;
#pragma unroll
      for (int kt = 0; kt < NT; ++kt) {
        floatx4 P;
#pragma unroll
        for (int r = 0; r < 4; ++r) P[r] = __builtin_amdgcn_exp2f(fmaf(S[kt][r], c2, nm));
        const bf16x4_t pb = __builtin_convertvector(P, bf16x4_t);
        if (kt & 1)
          Pb[kt / 2] = __builtin_shufflevector(prev, pb, 0, 1, 2, 3, 4, 5, 6, 7);  // keys 32 (kt / 2) ..
        else if (kt / 2 < kJ)
          prev = pb;
        else
          Pt = pb;  // the 16-key step (kTail)
      }

      // ---- O^T = V^T P^T: V operands of step j + 1 read during step j; the
      // row sums of the same bf16 P from the matrix core (ones x P^T) ----
      floatx4 O[kT], Ls = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < kT; ++t) O[t] = floatx4{0.f, 0.f, 0.f, 0.f};
      u32x4 vf[2][kT];
      auto vread = [&](int j, int buf) {
#pragma unroll
        for (int t = 0; t < kT; ++t) {
          const int d = dbase(t, qd);
          const u32x2 a = __builtin_bit_cast(u32x2, lds_tr(vb, v_off<DH>(32 * j + 4 * g4 + e, d)));
          const u32x2 b = __builtin_bit_cast(u32x2, lds_tr(vb, v_off<DH>(32 * j + 16 + 4 * g4 + e, d)));
          vf[buf][t] = u32x4{a[0], a[1], b[0], b[1]};
        }
      };
      vread(0, 0);
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        if (j + 1 < kJ) vread(j + 1, (j + 1) & 1);
#pragma unroll
        for (int t = 0; t < kT; ++t) {
          O[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vf[j & 1][t]), Pb[j], O[t], 0, 0, 0);
          ST_PIN_MFMA_LDS();
        }
        ST_BEFORE(ones8);
        Ls = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ones8), Pb[j], Ls, 0, 0, 0);
        ST_AFTER(Ls);
        ST_PIN_MFMA_LDS();
      }
      if (kTail) {  // keys 32 kJ .. 32 kJ + 15: v_mfma_f32_16x16x16_bf16
        short4_t vt[kT];
#pragma unroll
        for (int t = 0; t < kT; ++t) vt[t] = lds_tr(vb, v_off<DH>(32 * kJ + 4 * g4 + e, dbase(t, qd)));
#pragma unroll
        for (int t = 0; t < kT; ++t) {
          O[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[t], __builtin_bit_cast(short4_t, Pt), O[t], 0, 0, 0);
          ST_PIN_MFMA();
        }
        ST_BEFORE(ones4);
        Ls = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, ones4), __builtin_bit_cast(short4_t, Pt), Ls, 0, 0, 0);
        ST_AFTER(Ls);
        ST_PIN_MFMA();
      }
      const float inv = 1.0f / Ls[0];

      // ---- normalise and scatter: one 16-byte store per pair of output tiles ----
      if (qcode[i] != kPadSlot) {
        uint16_t* out = o + row_at(qtok[i], p.so) + hoff;
#pragma unroll
        for (int m2 = 0; m2 < kT / 2; ++m2) {
          const u32x2 a = __builtin_bit_cast(u32x2, __builtin_convertvector(O[2 * m2] * inv, bf16x4_t));
          const u32x2 b = __builtin_bit_cast(u32x2, __builtin_convertvector(O[2 * m2 + 1] * inv, bf16x4_t));
          const u32x4 w = odd ? u32x4{b[0], b[1], a[0], a[1]} : u32x4{a[0], a[1], b[0], b[1]};
          *reinterpret_cast<u32x4*>(out + 32 * m2 + 8 * g4) = w;
        }
      }
    }
  };
  if (cur.masked)
    tiles(std::true_type{});
  else
    tiles(std::false_type{});
}

// kernel parameters of a plan: nqb query blocks and nchunk key chunks per window
StreamParams make_params(const swin3d_wattn_plan* pl, const swin3d_wattn_strides_t* st, int nqb, int nchunk) {
  StreamParams p;
  p.g = make_geom(pl);
  p.nqb = nqb;
  p.nchunk = nchunk;
  p.n_windows = (int32_t)pl->n_windows;
  p.div_qb = make_fastdiv((uint32_t)nqb);
  p.sq = (uint32_t)st->q;
  p.sk = (uint32_t)st->k;
  p.sv = (uint32_t)st->v;
  p.so = (uint32_t)st->o;
  p.c2 = pl->c2;
  p.beta01 = (uint32_t)pl->beta_bf16[0] | ((uint32_t)pl->beta_bf16[1] << 16);
  p.beta2 = pl->beta_bf16[2];
  p.pad = pl->pad_bf16;
  const int64_t dh2 = 2 * (int64_t)pl->desc.head_dim;
  const bool off32 = st->k == st->v && pl->tokens <= (int64_t(1) << 24) && 2 * st->k < (int64_t(1) << 24) &&
                     (pl->tokens - 1) * 2 * st->k + dh2 < (int64_t(1) << 32);
  p.kv2 = off32 ? (uint32_t)(2 * st->k) : 0u;
  return p;
}

template <int DH, int WAVES, int KC, int QT>
hipError_t launch(const swin3d_wattn_plan* pl, const void* q, const void* k, const void* v, void* o,
                  const swin3d_wattn_strides_t* st, hipStream_t s) {
  constexpr int kQB = 16 * WAVES * QT;
  StreamParams p = make_params(pl, st, (pl->N + kQB - 1) / kQB, (pl->N + KC - 1) / KC);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  uint16_t* oo = static_cast<uint16_t*>(o);
  void* args[] = {&qq, &kk, &vv, &oo, &p};
  const dim3 grid((unsigned)((pl->n_windows + 7) / 8 * 8 * p.nqb), (unsigned)pl->desc.heads);
  // grids that need padding get the instance that skips query blocks and key
  // chunks of padding only
  const bool pad = pl->padded[0] != pl->desc.D || pl->padded[1] != pl->desc.H || pl->padded[2] != pl->desc.W;
  // and K/V within 32-bit byte offsets the instance with one multiply-add
  // per loaded row
  const void* fn = p.kv2 ? (pad ? reinterpret_cast<const void*>(&wattn_stream_item<DH, WAVES, KC, QT, true, true>)
                                : reinterpret_cast<const void*>(&wattn_stream_item<DH, WAVES, KC, QT, false, true>))
                         : (pad ? reinterpret_cast<const void*>(&wattn_stream_item<DH, WAVES, KC, QT, true, false>)
                                : reinterpret_cast<const void*>(&wattn_stream_item<DH, WAVES, KC, QT, false, false>));
  return hipLaunchKernel(fn, grid, dim3(64 * WAVES), args, 0, s);
}

template <int DH, int NT>
hipError_t launch_window(const swin3d_wattn_plan* pl, const void* q, const void* k, const void* v, void* o,
                         const swin3d_wattn_strides_t* st, hipStream_t s) {
  StreamParams p = make_params(pl, st, 1, 1);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  uint16_t* oo = static_cast<uint16_t*>(o);
  void* args[] = {&qq, &kk, &vv, &oo, &p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&wattn_window_item<DH, NT>),
                         dim3((unsigned)pl->n_windows, (unsigned)pl->desc.heads), dim3(256), args, 0, s);
}

}  // namespace

int wattn_launch_stream(const swin3d_wattn_plan* p, const void* q, const void* k, const void* v, void* o,
                        const swin3d_wattn_strides_t* stride, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool k48 = p->threads == 192;  // the plan's block shape: 3 waves and 48-key chunks
  hipError_t e;
  // two query tiles per wave at every head_dim: each K and V operand read
  // from LDS serves both
  if (p->desc.head_dim == 128)
    e = k48 ? launch<128, 3, 48, 2>(p, q, k, v, o, stride, s) : launch<128, 4, 64, 2>(p, q, k, v, o, stride, s);
  else if (p->desc.head_dim == 64)
    e = k48 ? launch<64, 3, 48, 2>(p, q, k, v, o, stride, s) : launch<64, 4, 64, 2>(p, q, k, v, o, stride, s);
  else
    e = k48 ? launch<32, 3, 48, 2>(p, q, k, v, o, stride, s) : launch<32, 4, 64, 2>(p, q, k, v, o, stride, s);
  return (int)e;
}

int wattn_launch_window(const swin3d_wattn_plan* p, const void* q, const void* k, const void* v, void* o,
                        const swin3d_wattn_strides_t* stride, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the plan admits N x head_dim = 18432 only: 144 x 128 or 288 x 64
  const hipError_t e = p->desc.head_dim == 128 ? launch_window<128, 9>(p, q, k, v, o, stride, s)
                                               : launch_window<64, 18>(p, q, k, v, o, stride, s);
  return (int)e;
}
