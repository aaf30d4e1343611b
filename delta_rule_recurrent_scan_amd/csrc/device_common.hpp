// Device helpers shared by the OSDN / GDN-2 kernels (gfx950, wave64).
//
// * bf16 <-> fp32 conversion (hardware round-to-nearest-even on gfx950),
// * an "NT" MFMA tile helper: acc(16x16, fp32) += A(16 x K) * B(16 x K)^T with
//   both operands read from LDS as K-contiguous rows,
// * wave-level reductions built from DPP row operations and the gfx950
//   cross-row lane swaps (no LDS round trip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace osdn {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// ---------------------------------------------------------------------------
// MFMA tile: acc[16x16] += A[16 x KEXT] * Bt[16 x KEXT]^T
//
// A and Bt point at the tile origin in LDS (row-major, leading dimensions lda
// and ldb elements). Output layout (all 16x16 fp32 MFMAs on CDNA): lane l holds
// rows 4*(l/16) + i, i = 0..3, of column l%16 in acc[i].
//
// Operand layout: lane l supplies row l%16 of A and of Bt and a run of K
// indices chosen by l/16. A and Bt use the same (lane group, slot) -> k map, so
// the product is independent of the order the hardware assigns within a run.
// ---------------------------------------------------------------------------
template <int KEXT>
__device__ __forceinline__ void mma_nt(f32x4& acc, const __bf16* A, int lda,
                                       const __bf16* Bt, int ldb) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const __bf16* a = A + r * lda;
  const __bf16* b = Bt + r * ldb;
#pragma unroll
  for (int kk = 0; kk + 32 <= KEXT; kk += 32) {
    bf16x8 av = *reinterpret_cast<const bf16x8*>(a + kk + g * 8);
    bf16x8 bv = *reinterpret_cast<const bf16x8*>(b + kk + g * 8);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
  }
  if constexpr (KEXT % 32 == 16) {
    constexpr int kk = KEXT - 16;
    bf16x4 av = *reinterpret_cast<const bf16x4*>(a + kk + g * 4);
    bf16x4 bv = *reinterpret_cast<const bf16x4*>(b + kk + g * 4);
    typedef __attribute__((ext_vector_type(4))) short s4;
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
        __builtin_bit_cast(s4, av), __builtin_bit_cast(s4, bv), acc, 0, 0, 0);
  }
  static_assert(KEXT % 16 == 0, "K extent must be a multiple of 16");
}

template <int KEXT>
__device__ __forceinline__ void mma_nt(f32x4& acc, const float* A, int lda,
                                       const float* Bt, int ldb) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const float* a = A + r * lda + g;
  const float* b = Bt + r * ldb + g;
#pragma unroll
  for (int kk = 0; kk < KEXT; kk += 4)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[kk], b[kk], acc, 0, 0, 0);
  static_assert(KEXT % 4 == 0, "K extent must be a multiple of 4");
}

// Operand fragment of a 16 x KEXT tile held in registers, loaded once from
// LDS (row l%16, k-run chosen by l/16, as in mma_nt) and reusable across
// several MFMAs.
template <int KEXT, typename Tin>
struct Frag;

template <int KEXT>
struct Frag<KEXT, __bf16> {
  static constexpr int N32 = KEXT / 32, R16 = (KEXT % 32) / 16;
  bf16x8 v[N32 > 0 ? N32 : 1];
  bf16x4 t;
  __device__ __forceinline__ void load(const __bf16* base, int ld) {
    load_row(base + (threadIdx.x & 15) * ld);
  }
  // `row` points at the start of this lane's row (row lane % 16 of the tile).
  __device__ __forceinline__ void load_row(const __bf16* row) {
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int i = 0; i < N32; ++i)
      v[i] = *reinterpret_cast<const bf16x8*>(row + 32 * i + g * 8);
    if constexpr (R16) t = *reinterpret_cast<const bf16x4*>(row + 32 * N32 + g * 4);
  }
  // The same fragment of the transpose of a KEXT x 16 block stored k-major
  // (row k holds 16 consecutive n), by the gfx950 LDS transpose read: within
  // each group of 16 lanes, lane s reads 4 consecutive n of row s/4 (plus the
  // group's row offset) at column 4*(s%4), and receives 4 consecutive k of
  // column s%16. Two reads give the 8 k of one 16x16x32 step in Frag's k
  // order. `base` points at element (k0, n0); ld is the row stride.
  __device__ __forceinline__ void load_kmajor(const __bf16* base, int ld) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, s = lane & 15;
    const __bf16* p = base + (s >> 2) * ld + 4 * (s & 3);
#pragma unroll
    for (int i = 0; i < N32; ++i) {
      const __bf16* q = p + (32 * i + 8 * g) * ld;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)q);
      const bf16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(q + 4 * ld));
      v[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    if constexpr (R16)
      t = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4*)(p + (32 * N32 + 4 * g) * ld));
  }
  // The same fragments in the permuted k order that accumulator tiles give
  // directly: in 32-wide step i, lane group g holds k = 32i + 4g + {0..3}
  // and 32i + 16 + 4g + {0..3} (the rows an accumulator lane holds in two
  // adjacent 16x16 tiles). Any k order serves a contraction as long as both
  // operands use it. Row-major source (row lane % 16, k along the row):
  __device__ __forceinline__ void load_perm(const __bf16* base, int ld) {
    const int lane = threadIdx.x & 63;
    const __bf16* p = base + (lane & 15) * ld + 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < N32; ++i) {
      const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p + 32 * i);
      const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 32 * i + 16);
      v[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    if constexpr (R16) t = *reinterpret_cast<const bf16x4*>(p + 32 * N32);
  }
  // k-major source (as load_kmajor), permuted k order.
  __device__ __forceinline__ void load_kmajor_perm(const __bf16* base, int ld) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, s = lane & 15;
    const __bf16* p = base + (s >> 2) * ld + 4 * (s & 3) + 4 * g * ld;
#pragma unroll
    for (int i = 0; i < N32; ++i) {
      const __bf16* q = p + 32 * i * ld;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)q);
      const bf16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(q + 16 * ld));
      v[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    if constexpr (R16)
      t = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 32 * N32 * ld));
  }
  // Fragment-major global storage (ELEMS elements): slot s of lane l at
  // [s][l], so that a wave moves each slot as one contiguous block.
  static constexpr int ELEMS = 16 * KEXT;
  // Accumulator tile b (16 k values) of a permuted-order fragment, stored
  // in place: tiles 2i and 2i + 1 fill the low and high halves of step i.
  __device__ __forceinline__ static void store_acc_tile(__bf16* base, int b, const f32x4& a) {
    bf16x4 h;
    h[0] = (__bf16)a[0]; h[1] = (__bf16)a[1]; h[2] = (__bf16)a[2]; h[3] = (__bf16)a[3];
    const int lane = threadIdx.x & 63;
    __bf16* d = (b >> 1) < N32 ? base + ((b >> 1) * 64 + lane) * 8 + 4 * (b & 1)
                               : base + N32 * 512 + lane * 4;
    *reinterpret_cast<bf16x4*>(d) = h;
  }
  // One element (accumulator value i) of store_acc_tile.
  __device__ __forceinline__ static void store_acc_elem(__bf16* base, int b, int i, float a) {
    const int lane = threadIdx.x & 63;
    __bf16* d = (b >> 1) < N32 ? base + ((b >> 1) * 64 + lane) * 8 + 4 * (b & 1)
                               : base + N32 * 512 + lane * 4;
    d[i] = (__bf16)a;
  }
  // Accumulator tile formed transposed over this fragment's 16 rows (lane
  // l holds row l % 16, k = 16 cb + 4 (l / 16) + {0..3}), rounded and stored
  // straight into the layout of store_global: the four values are one
  // contiguous half of a lane's 16-byte slot.
  __device__ __forceinline__ static void store_acc_kblock(__bf16* base, int cb,
                                                          const f32x4& a) {
    bf16x4 h;
    h[0] = (__bf16)a[0]; h[1] = (__bf16)a[1]; h[2] = (__bf16)a[2]; h[3] = (__bf16)a[3];
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    __bf16* d = (cb >> 1) < N32
                    ? base + (((cb >> 1) * 64 + ((cb & 1) * 2 + (g >> 1)) * 16 + r) * 8 +
                              4 * (g & 1))
                    : base + N32 * 512 + (g * 16 + r) * 4;
    *reinterpret_cast<bf16x4*>(d) = h;
  }
  __device__ __forceinline__ void store_global(__bf16* base) const {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < N32; ++i)
      *reinterpret_cast<bf16x8*>(base + (i * 64 + lane) * 8) = v[i];
    if constexpr (R16)
      *reinterpret_cast<bf16x4*>(base + N32 * 512 + lane * 4) = t;
  }
  __device__ __forceinline__ void load_global(const __bf16* base) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < N32; ++i)
      v[i] = *reinterpret_cast<const bf16x8*>(base + (i * 64 + lane) * 8);
    if constexpr (R16)
      t = *reinterpret_cast<const bf16x4*>(base + N32 * 512 + lane * 4);
  }
};

template <int KEXT>
struct Frag<KEXT, float> {
  float v[KEXT / 4];
  __device__ __forceinline__ void load(const float* base, int ld) {
    load_row(base + (threadIdx.x & 15) * ld);
  }
  __device__ __forceinline__ void load_row(const float* row) {
    const float* p = row + ((threadIdx.x & 63) >> 4);
#pragma unroll
    for (int i = 0; i < KEXT / 4; ++i) v[i] = p[4 * i];
  }
  // Transpose of a KEXT x 16 block stored k-major: lane l takes column l%16
  // of rows 4i + l/16.
  __device__ __forceinline__ void load_kmajor(const float* base, int ld) {
    const int lane = threadIdx.x & 63;
    const float* p = base + (lane >> 4) * ld + (lane & 15);
#pragma unroll
    for (int i = 0; i < KEXT / 4; ++i) v[i] = p[4 * i * ld];
  }
  // Permuted k order (see the bf16 fragment): step 4b + i, lane group g
  // holds k = 16b + 4g + i, i.e. accumulator value i of tile b.
  __device__ __forceinline__ void load_perm(const float* base, int ld) {
    const int lane = threadIdx.x & 63;
    const float* p = base + (lane & 15) * ld + 4 * (lane >> 4);
#pragma unroll
    for (int b = 0; b < KEXT / 16; ++b) {
      const float4 x = *reinterpret_cast<const float4*>(p + 16 * b);
      v[4 * b] = x.x; v[4 * b + 1] = x.y; v[4 * b + 2] = x.z; v[4 * b + 3] = x.w;
    }
  }
  __device__ __forceinline__ void load_kmajor_perm(const float* base, int ld) {
    const int lane = threadIdx.x & 63;
    const float* p = base + 4 * (lane >> 4) * ld + (lane & 15);
#pragma unroll
    for (int b = 0; b < KEXT / 16; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * b + i] = p[(16 * b + i) * ld];
  }
  static constexpr int ELEMS = 16 * KEXT;
  __device__ __forceinline__ static void store_acc_tile(float* base, int b, const f32x4& a) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i) base[(4 * b + i) * 64 + lane] = a[i];
  }
  __device__ __forceinline__ static void store_acc_elem(float* base, int b, int i, float a) {
    base[(4 * b + i) * 64 + (threadIdx.x & 63)] = a;
  }
  // As the bf16 fragment's: the accumulator tile over the fragment's 16
  // rows at 16-wide k block cb, into the layout of store_global.
  __device__ __forceinline__ static void store_acc_kblock(float* base, int cb,
                                                          const f32x4& a) {
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) base[(4 * cb + g) * 64 + i * 16 + r] = a[i];
  }
  __device__ __forceinline__ void store_global(float* base) const {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < KEXT / 4; ++i) base[i * 64 + lane] = v[i];
  }
  __device__ __forceinline__ void load_global(const float* base) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < KEXT / 4; ++i) v[i] = base[i * 64 + lane];
  }
};

// A 16x16 fp32 accumulator tile in global memory in accumulator order (lane
// l's four values contiguous at [l][0..3]), rounded to Tin.
__device__ __forceinline__ void acc_store(const f32x4& a, __bf16* base) {
  bf16x4 b;
  b[0] = (__bf16)a[0]; b[1] = (__bf16)a[1]; b[2] = (__bf16)a[2]; b[3] = (__bf16)a[3];
  *reinterpret_cast<bf16x4*>(base + (threadIdx.x & 63) * 4) = b;
}
__device__ __forceinline__ void acc_store(const f32x4& a, float* base) {
  *reinterpret_cast<f32x4*>(base + (threadIdx.x & 63) * 4) = a;
}
__device__ __forceinline__ f32x4 acc_load(const __bf16* base) {
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(base + (threadIdx.x & 63) * 4);
  return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}
__device__ __forceinline__ f32x4 acc_load(const float* base) {
  return *reinterpret_cast<const f32x4*>(base + (threadIdx.x & 63) * 4);
}

// acc += A * B^T from two register fragments.
template <int KEXT>
__device__ __forceinline__ void mma(f32x4& acc, const Frag<KEXT, __bf16>& a,
                                    const Frag<KEXT, __bf16>& b) {
#pragma unroll
  for (int i = 0; i < Frag<KEXT, __bf16>::N32; ++i)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v[i], b.v[i], acc, 0, 0, 0);
  if constexpr (Frag<KEXT, __bf16>::R16) {
    typedef __attribute__((ext_vector_type(4))) short s4;
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
        __builtin_bit_cast(s4, a.t), __builtin_bit_cast(s4, b.t), acc, 0, 0, 0);
  }
}

template <int KEXT>
__device__ __forceinline__ void mma(f32x4& acc, const Frag<KEXT, float>& a,
                                    const Frag<KEXT, float>& b) {
#pragma unroll
  for (int i = 0; i < KEXT / 4; ++i)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
}

// Orders this wave's earlier LDS writes before its later LDS reads (data
// exchanged between lanes of one wave needs no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// v, or zeros when !keep. Selected per component: a select of the whole
// struct becomes a select of addresses, which forces the register arrays it
// reads into scratch memory.
__device__ __forceinline__ uint4 keep_or_zero(const uint4& v, bool keep) {
  return uint4{keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u};
}

// Index of this thread's wave in the workgroup as a wave-uniform value, so
// that the compiler keeps indexing derived from it in scalar registers.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Row (within a 16x16 output tile) of element i held by this lane.
__device__ __forceinline__ int acc_row(int i) { return 4 * ((threadIdx.x & 63) >> 4) + i; }
__device__ __forceinline__ int acc_col() { return threadIdx.x & 15; }

// ---------------------------------------------------------------------------
// Wave reductions
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                         0xf, 0xf, false));
}

// Sum over each row of 16 lanes; every lane of the row receives the row sum.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  return x;
}

// x + (x of lane l^16): rows 0/1 and 2/3 exchange their values.
// (The two results of the swap are read into scalars before the bit cast: a
// bit cast applied directly to an element of the returned vector reads
// element 0.)
__device__ __forceinline__ float add_swap16(float x) {
  const unsigned u = __float_as_uint(x);
  const auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned lo = s[0], hi = s[1];
  return __uint_as_float(lo) + __uint_as_float(hi);
}

// x + (x of lane l^32): the two 32-lane halves exchange their values.
__device__ __forceinline__ float add_swap32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned lo = s[0], hi = s[1];
  return __uint_as_float(lo) + __uint_as_float(hi);
}

// Sum over aligned groups of L consecutive lanes (L = 2, 4, ..., 64); every
// lane of a group receives the group's sum.
template <int L>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(L == 2 || L == 4 || L == 8 || L == 16 || L == 32 || L == 64,
                "group size");
  x += dpp_f<0xB1>(x);
  if constexpr (L >= 4) x += dpp_f<0x4E>(x);
  if constexpr (L >= 8) x += dpp_f<0x141>(x);
  if constexpr (L >= 16) x += dpp_f<0x140>(x);
  if constexpr (L >= 32) x = add_swap16(x);
  if constexpr (L >= 64) x = add_swap32(x);
  return x;
}

// Sum over the lanes that share l % P (P = 2, 4, 8, 16); every lane
// receives the sum of its class. Rotations within each row of 16 lanes, then
// the cross-row swaps.
template <int P>
__device__ __forceinline__ float strided_sum(float x) {
  static_assert(P == 2 || P == 4 || P == 8 || P == 16, "stride");
  if constexpr (P == 2) x += dpp_f<0x122>(x);  // row_ror:2
  if constexpr (P <= 4) x += dpp_f<0x124>(x);  // row_ror:4
  if constexpr (P <= 8) x += dpp_f<0x128>(x);  // row_ror:8
  return add_swap32(add_swap16(x));
}

// Inclusive prefix sum over the 64 lanes of a wave (lane l gets the sum of
// lanes 0..l), by log-step shuffles.
__device__ __forceinline__ float wave_prefix_sum(float x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// Sum over all 64 lanes; every lane receives the total.
__device__ __forceinline__ float wave_sum(float x) {
  return add_swap32(add_swap16(row16_sum(x)));
}

}  // namespace osdn
