// Register layout of a (batch, head) state held by one workgroup of 256
// threads for the token-recurrent kernels (decode and backward): a state row
// is spread over an aligned group of 16 lanes ("column lanes"), each holding
// D/16 of its columns as 16-byte pieces 64 columns apart (so each load
// instruction of a group covers 256 contiguous bytes of the row); the 16 row
// groups of the workgroup take rows g, g + 16, ... Reductions along a row are
// row-of-16 DPP sums.
#pragma once

#include "device_common.hpp"

namespace osdn {

constexpr int kDecThreads = 256;

// Column of the j-th value held by column lane cl, for rows of D values.
template <int D>
__device__ __forceinline__ int dec_col(int cl, int j) {
  constexpr int N = D / 16;
  if constexpr (N >= 4) return 4 * cl + 64 * (j >> 2) + (j & 3);
  else return N * cl + j;
}

// The D/16 values of one row that column lane cl holds, widened to fp32.
template <int D, typename Tin>
__device__ __forceinline__ void load_cols(const Tin* row, int cl, float (&x)[D / 16]) {
  constexpr int N = D / 16;
  if constexpr (N >= 4) {
#pragma unroll
    for (int m = 0; m < N / 4; ++m) {
      const Tin* p = row + 4 * cl + 64 * m;
      if constexpr (sizeof(Tin) == 4) {
        const float4 f = *reinterpret_cast<const float4*>(p);
        x[4 * m + 0] = f.x; x[4 * m + 1] = f.y; x[4 * m + 2] = f.z; x[4 * m + 3] = f.w;
      } else {
        const uint2 u = *reinterpret_cast<const uint2*>(p);
        const Tin* h = reinterpret_cast<const Tin*>(&u);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * m + e] = to_f32(h[e]);
      }
    }
  } else {
    const Tin* p = row + N * cl;
    if constexpr (sizeof(Tin) == 4) {
      const float2 f = *reinterpret_cast<const float2*>(p);
      x[0] = f.x; x[1] = f.y;
    } else {
      const unsigned u = *reinterpret_cast<const unsigned*>(p);
      const Tin* h = reinterpret_cast<const Tin*>(&u);
      x[0] = to_f32(h[0]); x[1] = to_f32(h[1]);
    }
  }
}

template <int D>
__device__ __forceinline__ void store_cols(float* row, int cl, const float (&x)[D / 16]) {
  constexpr int N = D / 16;
  if constexpr (N >= 4) {
#pragma unroll
    for (int m = 0; m < N / 4; ++m)
      *reinterpret_cast<float4*>(row + 4 * cl + 64 * m) =
          float4{x[4 * m], x[4 * m + 1], x[4 * m + 2], x[4 * m + 3]};
  } else {
    *reinterpret_cast<float2*>(row + N * cl) = float2{x[0], x[1]};
  }
}

}  // namespace osdn
