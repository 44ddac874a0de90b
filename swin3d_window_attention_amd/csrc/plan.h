// Internal plan shared by the host API and the kernel launchers.
#pragma once
#include <stdint.h>

#include "swin3d_wattn.h"

struct swin3d_wattn_plan {
  swin3d_wattn_desc_t desc;
  int32_t padded[3];
  int32_t nwin[3];          // windows per axis
  int64_t n_windows;        // B * nwin[0] * nwin[1] * nwin[2]
  int64_t n_masked_windows; // windows with a region cut or padding
  int32_t N;                // tokens per window
  int64_t tokens;           // B * D * H * W
  int64_t elems;            // tokens * heads * head_dim
  int32_t elem_bytes;
  int32_t kernel;           // 1: bf16 MFMA (N = 144, dh 64), 2: f32 split-bf16 MFMA,
                            // 3: bf16 MFMA with K/V streamed (any N, dh 32, 64 or 128),
                            // 4: f32 MFMA (N <= 256, dh 32 or 64),
                            // 5: bf16 MFMA, whole window in LDS (N x dh = 144 x 128 or 288 x 64)
  int64_t workgroups;       // workgroups one run launches
  int32_t threads;          // threads per workgroup
  float c2;                 // scale * log2(e)
  float bias2;              // cross_region_bias * log2(e)
  // bf16 kernel: the cross-region bias divided by scale, split into three
  // bf16 terms whose sum is exact to float precision, and the padding-key
  // offset (-2^100: its exponential underflows to exactly zero)
  uint16_t beta_bf16[3];
  uint16_t pad_bf16;
  // per axis: window indices that hold a region cut or padding (-1 = none)
  int32_t special[3][3];
  // per axis: window indices that hold padding (-1 = none); padding spans
  // fewer positions than a window, so at most two windows per axis
  int32_t padwin[3][2];
};

// Kernel launchers (wattn_bf16.hip, wattn_f32x3.hip, wattn_stream.hip for
// the streaming and the whole-window kernels, wattn_f32m.hip).
// Each launches its kernel for the plan on `stream` (a hipStream_t) and
// returns the HIP runtime's status (0 = success). `stride` holds the token
// strides of Q, K, V and O in elements, already validated.
int wattn_launch_bf16(const swin3d_wattn_plan* p, const void* q, const void* k, const void* v, void* o,
                      const swin3d_wattn_strides_t* stride, void* stream);
int wattn_launch_f32x3(const swin3d_wattn_plan* p, const void* q, const void* k, const void* v, void* o,
                       const swin3d_wattn_strides_t* stride, void* stream);
int wattn_launch_stream(const swin3d_wattn_plan* p, const void* q, const void* k, const void* v, void* o,
                        const swin3d_wattn_strides_t* stride, void* stream);
int wattn_launch_window(const swin3d_wattn_plan* p, const void* q, const void* k, const void* v, void* o,
                        const swin3d_wattn_strides_t* stride, void* stream);
int wattn_launch_f32m(const swin3d_wattn_plan* p, const void* q, const void* k, const void* v, void* o,
                      const swin3d_wattn_strides_t* stride, void* stream);
// adaln.hip: the fused AdaLN + residual kernel for an already validated desc.
int adaln_launch(const swin3d_adaln_desc_t* d, const void* x, const void* res, const float* gamma,
                 const float* beta, void* out, void* stream);
