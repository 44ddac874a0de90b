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
  int32_t kernel;           // 0: f32 VALU, 1: bf16 MFMA
  int64_t workgroups;
  int32_t threads;
  float c2;                 // scale * log2(e)
  float bias2;              // cross_region_bias * log2(e)
};

// Defined in kernels.hip. Launches the plan's kernel; returns a swin3d code.
int swin3d_wattn_launch(const swin3d_wattn_plan* p, const void* q, const void* k, const void* v,
                        void* o, void* stream);
