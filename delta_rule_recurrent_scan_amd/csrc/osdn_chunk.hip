// Phase 2 of the OSDN forward: the chunkwise WY delta rule with the
// preconditioned keys K~ in place of K.
//
// [OSDN-it] section 2.1: the OSDN write S_t = S_{t-1} + beta_t (v_t - S_{t-1}k_t)
// k~_t^T keeps DeltaNet's chunk-parallel WY pipeline, with K~ replacing K in the
// chunk Gram matrix and in the intra-chunk scores. Per chunk of C tokens with
// entry state S0 (Dv x Dk):
//   A   = strictLower(diag(beta) K K~^T)                 (chunk Gram, C x C)
//   T   = (I + A)^-1                                     (unit lower triangular)
//   W   = T diag(beta) (V - K S0^T)                      (C x Dv)
//   O   = Q S0^T + (Q K~^T masked to i <= t) W           (inclusive readout)
//   S1  = S0 + W^T K~
// This is the token recurrence rewritten exactly: row t of W is
// beta_t (v_t - S_{t-1} k_t).
//
// One workgroup (4 waves) owns one (batch, head) and one tile of VT value
// columns, and walks the chunks in order with its VT x Dk slice of the state
// held in fp32 MFMA accumulators. Rows of S evolve independently given K, K~
// and beta, so value tiles need no communication; the V-independent chunk
// quantities (A, T, Q K~^T) are recomputed by each tile's workgroup instead of
// being written to and re-read from HBM.
//
// Products run on MFMA in the operand dtype (bf16 in, fp32 accumulate; or fp32
// in for the fp32 path); the triangular inverse is fp32 forward substitution in
// LDS on 16x16 diagonal blocks followed by blocked off-diagonal updates.
#include "device_common.hpp"
#include "launch.hpp"

namespace osdn {

template <int DK, int C, int VT, typename Tin>
struct ChunkCfg {
  static constexpr int NW = 4, NT = 256;
  static constexpr int PAD = sizeof(Tin) == 2 ? 8 : 4;
  static constexpr int LDK = DK + PAD;  // rows of Dk elements
  static constexpr int LDC = C + PAD;   // rows of C elements (operand dtype)
  static constexpr int LDF = C + 4;     // rows of C fp32 elements
  static constexpr int TB = C / 16, VB = VT / 16, DB = DK / 16;
  static constexpr int VEC = 16 / sizeof(Tin);  // elements per 16-byte load
  static constexpr size_t oK = 0;
  static constexpr size_t oQ = oK + (size_t)C * LDK * sizeof(Tin);
  static constexpr size_t oKT = oQ + (size_t)C * LDK * sizeof(Tin);
  static constexpr size_t oKTt = oKT + (size_t)C * LDK * sizeof(Tin);
  static constexpr size_t oS = oKTt + (size_t)DK * LDC * sizeof(Tin);
  static constexpr size_t oV = oS + (size_t)VT * LDK * sizeof(Tin);
  static constexpr size_t oB = oV + (size_t)C * VT * sizeof(Tin);
  static constexpr size_t oA = oB + (size_t)C * 4;
  static constexpr size_t oTf = oA + (size_t)C * LDF * 4;
  static constexpr size_t oY = oTf + (size_t)C * LDF * 4;
  static constexpr size_t oTb = oY + (size_t)(TB > 1 ? TB - 1 : 1) * 256 * 4;
  static constexpr size_t oP = oTb + (size_t)C * LDC * sizeof(Tin);
  static constexpr size_t oR = oP + (size_t)C * LDC * sizeof(Tin);
  static constexpr size_t oW = oR + (size_t)VT * LDC * sizeof(Tin);
  static constexpr size_t bytes = oW + (size_t)VT * LDC * sizeof(Tin);
  static constexpr bool fits = bytes <= 163840;
  static constexpr int NS = (VB * DB + NW - 1) / NW;  // state tiles per wave
  static constexpr int NO = (TB * VB + NW - 1) / NW;  // output tiles per wave
};

template <int DK, int C, int VT, typename Tin>
__global__ __launch_bounds__(256) void osdn_chunk_kernel(
    int BH, int T, int Dv, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ ktil, const Tin* __restrict__ v,
    const float* __restrict__ beta, const float* __restrict__ S0, float scale,
    Tin* __restrict__ o, float* __restrict__ ST) {
  using G = ChunkCfg<DK, C, VT, Tin>;
  constexpr int LDK = G::LDK, LDC = G::LDC, LDF = G::LDF;
  constexpr int TB = G::TB, VB = G::VB, DB = G::DB, VEC = G::VEC;
  __shared__ __attribute__((aligned(16))) unsigned char smem[G::bytes];
  Tin* Ks = reinterpret_cast<Tin*>(smem + G::oK);
  Tin* Qs = reinterpret_cast<Tin*>(smem + G::oQ);
  Tin* KTs = reinterpret_cast<Tin*>(smem + G::oKT);
  Tin* KTt = reinterpret_cast<Tin*>(smem + G::oKTt);
  Tin* Ss = reinterpret_cast<Tin*>(smem + G::oS);
  Tin* Vs = reinterpret_cast<Tin*>(smem + G::oV);
  float* bs = reinterpret_cast<float*>(smem + G::oB);
  float* Am = reinterpret_cast<float*>(smem + G::oA);
  float* Tf = reinterpret_cast<float*>(smem + G::oTf);
  float* Yb = reinterpret_cast<float*>(smem + G::oY);
  Tin* Tb = reinterpret_cast<Tin*>(smem + G::oTb);
  Tin* Pb = reinterpret_cast<Tin*>(smem + G::oP);
  Tin* Rt = reinterpret_cast<Tin*>(smem + G::oR);
  Tin* Wt = reinterpret_cast<Tin*>(smem + G::oW);

  const int nvt = Dv / VT;
  // XCD-aware order: workgroups are spread round-robin over the 8 XCDs, so
  // renumber them so that all value tiles of one (batch, head), which read the
  // same K, K~ and Q, run on the same XCD and share its L2.
  int lin = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) lin = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int bh = lin / nvt, vt = lin - bh * nvt;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int v0 = vt * VT;
  const size_t row0 = (size_t)bh * T;

  // Strictly-upper 16x16 blocks of T and P stay zero for the whole run.
  for (int e = tid; e < C * C; e += G::NT) {
    const int rr = e / C, cc = e % C;
    if ((cc >> 4) > (rr >> 4)) {
      Tb[rr * LDC + cc] = from_f32<Tin>(0.f);
      Pb[rr * LDC + cc] = from_f32<Tin>(0.f);
    }
  }

  // Persistent state slice, fp32, in MFMA accumulator layout.
  f32x4 Sacc[G::NS];
#pragma unroll
  for (int s = 0; s < G::NS; ++s) {
    const int job = wave + G::NW * s;
    const int vb = job / DB, db = job % DB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = 0.f;
      if (job < VB * DB && S0)
        x = S0[((size_t)bh * Dv + v0 + vb * 16 + acc_row(i)) * DK + db * 16 +
               acc_col()];
      Sacc[s][i] = x;
    }
    if (job < VB * DB) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Ss[(vb * 16 + acc_row(i)) * LDK + db * 16 + acc_col()] =
            from_f32<Tin>(Sacc[s][i]);
    }
  }

  const int nchunks = (T + C - 1) / C;
  for (int j = 0; j < nchunks; ++j) {
    const size_t t0 = row0 + (size_t)j * C;
    // ---- stage 1: chunk operands into LDS ---------------------------------
    // Rows past the end of the sequence (ragged last chunk) are zero: with
    // beta = 0 and k~ = 0 they change neither W nor S, and their outputs are
    // not stored.
    const int valid = min(C, T - j * C);
    for (int e = tid; e < C * DK / VEC; e += G::NT) {
      const int rr = e / (DK / VEC), cc = (e % (DK / VEC)) * VEC;
      uint4 kv = {0u, 0u, 0u, 0u}, qv = kv, tv = kv;
      if (rr < valid) {
        const size_t g = (t0 + rr) * DK + cc;
        kv = *reinterpret_cast<const uint4*>(k + g);
        qv = *reinterpret_cast<const uint4*>(q + g);
        tv = *reinterpret_cast<const uint4*>(ktil + g);
      }
      *reinterpret_cast<uint4*>(Ks + rr * LDK + cc) = kv;
      *reinterpret_cast<uint4*>(Qs + rr * LDK + cc) = qv;
      *reinterpret_cast<uint4*>(KTs + rr * LDK + cc) = tv;
      const Tin* te = reinterpret_cast<const Tin*>(&tv);
#pragma unroll
      for (int u = 0; u < VEC; ++u) KTt[(cc + u) * LDC + rr] = te[u];
    }
    for (int e = tid; e < C * VT / VEC; e += G::NT) {
      const int rr = e / (VT / VEC), cc = (e % (VT / VEC)) * VEC;
      uint4 vv = {0u, 0u, 0u, 0u};
      if (rr < valid)
        vv = *reinterpret_cast<const uint4*>(v + (t0 + rr) * Dv + v0 + cc);
      *reinterpret_cast<uint4*>(Vs + rr * VT + cc) = vv;
    }
    if (tid < C) bs[tid] = tid < valid ? beta[t0 + tid] : 0.f;
    __syncthreads();

    // ---- stage 2: Gram A, scores P, K S0^T -> RHS, Q S0^T -> O -------------
    constexpr int NL = TB * (TB + 1) / 2;  // lower-triangular 16x16 tiles
    for (int job = wave; job < 2 * NL + TB * VB; job += G::NW) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (job < 2 * NL) {
        const bool isP = job >= NL;
        int l = isP ? job - NL : job, a = 0;
        while (l > a) { l -= a + 1; ++a; }
        const int b = l;
        mma_nt<DK>(acc, (isP ? Qs : Ks) + a * 16 * LDK, LDK, KTs + b * 16 * LDK,
                   LDK);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = a * 16 + acc_row(i), cc = b * 16 + acc_col();
          if (isP)
            Pb[rr * LDC + cc] = from_f32<Tin>(cc <= rr ? acc[i] : 0.f);
          else
            Am[rr * LDF + cc] = cc < rr ? bs[rr] * acc[i] : 0.f;
        }
      } else {
        const int l = job - 2 * NL, tb = l / VB, vb = l % VB;
        mma_nt<DK>(acc, Ks + tb * 16 * LDK, LDK, Ss + vb * 16 * LDK, LDK);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = tb * 16 + acc_row(i), cc = vb * 16 + acc_col();
          Rt[cc * LDC + rr] =
              from_f32<Tin>(bs[rr] * (to_f32(Vs[rr * VT + cc]) - acc[i]));
        }
      }
    }
    f32x4 Oacc[G::NO];
#pragma unroll
    for (int s = 0; s < G::NO; ++s) {
      Oacc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int job = wave + G::NW * s;
      if (job < TB * VB) {
        const int tb = job / VB, vb = job % VB;
        mma_nt<DK>(Oacc[s], Qs + tb * 16 * LDK, LDK, Ss + vb * 16 * LDK, LDK);
      }
    }
    __syncthreads();

    // ---- stage 3: T = (I + A)^-1, fp32 ------------------------------------
    // Diagonal 16x16 blocks: thread (block b, column c) solves one column by
    // forward substitution.
    if (tid < 16 * TB) {
      const int b = tid >> 4, c = tid & 15;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = (i == c) ? 1.f : 0.f;
        const float* arow = Am + (b * 16 + i) * LDF + b * 16;
#pragma unroll
        for (int m = 0; m < i; ++m) s -= arow[m] * x[m];
        x[i] = s;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        Tf[(b * 16 + i) * LDF + b * 16 + c] = x[i];
        Tb[(b * 16 + i) * LDC + b * 16 + c] = from_f32<Tin>(x[i]);
      }
    }
    __syncthreads();
    // Off-diagonal blocks, one block row at a time:
    //   T_ab = -T_aa * sum_{c=b}^{a-1} A_ac T_cb.
    for (int a = 1; a < TB; ++a) {
      for (int e = tid; e < a * 256; e += G::NT) {
        const int b = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
        const float* arow = Am + (a * 16 + rr) * LDF;
        float s = 0.f;
        for (int m = b * 16; m < a * 16; ++m) s += arow[m] * Tf[m * LDF + b * 16 + cc];
        Yb[(b * 16 + rr) * 16 + cc] = s;
      }
      __syncthreads();
      for (int e = tid; e < a * 256; e += G::NT) {
        const int b = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
        const float* trow = Tf + (a * 16 + rr) * LDF + a * 16;
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m) s -= trow[m] * Yb[(b * 16 + m) * 16 + cc];
        Tf[(a * 16 + rr) * LDF + b * 16 + cc] = s;
        Tb[(a * 16 + rr) * LDC + b * 16 + cc] = from_f32<Tin>(s);
      }
      __syncthreads();
    }

    // ---- stage 4: W = T * RHS -> W^T in LDS --------------------------------
    for (int job = wave; job < TB * VB; job += G::NW) {
      const int tb = job / VB, vb = job % VB;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mma_nt<C>(acc, Tb + tb * 16 * LDC, LDC, Rt + vb * 16 * LDC, LDC);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Wt[(vb * 16 + acc_col()) * LDC + tb * 16 + acc_row(i)] = from_f32<Tin>(acc[i]);
    }
    __syncthreads();

    // ---- stage 5: O += P W (store), S += W^T K~ ----------------------------
#pragma unroll
    for (int s = 0; s < G::NO; ++s) {
      const int job = wave + G::NW * s;
      if (job < TB * VB) {
        const int tb = job / VB, vb = job % VB;
        mma_nt<C>(Oacc[s], Pb + tb * 16 * LDC, LDC, Wt + vb * 16 * LDC, LDC);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = tb * 16 + acc_row(i);
          if (rr < valid)
            o[(t0 + rr) * Dv + v0 + vb * 16 + acc_col()] =
                from_f32<Tin>(scale * Oacc[s][i]);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < G::NS; ++s) {
      const int job = wave + G::NW * s;
      if (job < VB * DB) {
        const int vb = job / DB, db = job % DB;
        mma_nt<C>(Sacc[s], Wt + vb * 16 * LDC, LDC, KTt + db * 16 * LDC, LDC);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Ss[(vb * 16 + acc_row(i)) * LDK + db * 16 + acc_col()] =
              from_f32<Tin>(Sacc[s][i]);
      }
    }
    __syncthreads();
  }

  if (ST) {
#pragma unroll
    for (int s = 0; s < G::NS; ++s) {
      const int job = wave + G::NW * s;
      if (job < VB * DB) {
        const int vb = job / DB, db = job % DB;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ST[((size_t)bh * Dv + v0 + vb * 16 + acc_row(i)) * DK + db * 16 +
             acc_col()] = Sacc[s][i];
      }
    }
  }
}

template <int DK, int C, int VT, typename Tin>
static int launch_cfg(const ChunkArgs& a, hipStream_t s) {
  if constexpr (!ChunkCfg<DK, C, VT, Tin>::fits) {
    return -1;
  } else {
    const int BH = a.B * a.H;
    dim3 grid(BH * (a.Dv / VT)), block(256);
    hipLaunchKernelGGL((osdn_chunk_kernel<DK, C, VT, Tin>), grid, block, 0, s,
                       BH, a.T, a.Dv, (const Tin*)a.q, (const Tin*)a.k,
                       (const Tin*)a.ktilde, (const Tin*)a.v, a.beta, a.S0,
                       a.scale, (Tin*)a.o, a.ST);
    return (int)hipGetLastError();
  }
}

// Value-tile width: 32 columns when that already gives at least one
// workgroup per compute unit, else 16 for more parallelism.
static int pick_vt(int BH, int Dv) { return (BH * (Dv / 32) >= 256) ? 32 : 16; }

template <int DK, int C, typename Tin>
static int launch_c(const ChunkArgs& a, hipStream_t s) {
  if (pick_vt(a.B * a.H, a.Dv) == 32) return launch_cfg<DK, C, 32, Tin>(a, s);
  return launch_cfg<DK, C, 16, Tin>(a, s);
}

template <int DK, typename Tin>
static int launch_dk(const ChunkArgs& a, hipStream_t s) {
  switch (a.chunk) {
    case 16: return launch_c<DK, 16, Tin>(a, s);
    case 32: return launch_c<DK, 32, Tin>(a, s);
    case 64: return launch_c<DK, 64, Tin>(a, s);
  }
  return -1;
}

int launch_osdn_chunk(const ChunkArgs& a, hipStream_t s) {
  if (a.bf16) {
    switch (a.Dk) {
      case 32: return launch_dk<32, __bf16>(a, s);
      case 64: return launch_dk<64, __bf16>(a, s);
      case 128: return launch_dk<128, __bf16>(a, s);
    }
  } else {
    switch (a.Dk) {
      case 32: return launch_dk<32, float>(a, s);
      case 64: return launch_dk<64, float>(a, s);
      case 128: return launch_dk<128, float>(a, s);
    }
  }
  return -1;
}

template <int DK, typename Tin>
static bool fits_dk(int chunk) {
  // Both value-tile widths must fit, since the width depends on B*H at launch.
  switch (chunk) {
    case 16: return ChunkCfg<DK, 16, 32, Tin>::fits && ChunkCfg<DK, 16, 16, Tin>::fits;
    case 32: return ChunkCfg<DK, 32, 32, Tin>::fits && ChunkCfg<DK, 32, 16, Tin>::fits;
    case 64: return ChunkCfg<DK, 64, 32, Tin>::fits && ChunkCfg<DK, 64, 16, Tin>::fits;
  }
  return false;
}

bool osdn_chunk_supported(int Dk, int chunk, int bf16) {
  if (bf16) {
    switch (Dk) {
      case 32: return fits_dk<32, __bf16>(chunk);
      case 64: return fits_dk<64, __bf16>(chunk);
      case 128: return fits_dk<128, __bf16>(chunk);
    }
  } else {
    switch (Dk) {
      case 32: return fits_dk<32, float>(chunk);
      case 64: return fits_dk<64, float>(chunk);
      case 128: return fits_dk<128, float>(chunk);
    }
  }
  return false;
}

}  // namespace osdn
