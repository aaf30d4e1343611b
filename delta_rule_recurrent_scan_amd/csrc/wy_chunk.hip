// Chunkwise WY delta-rule engine (phase 2 of the OSDN forward).
//
// One engine serves every update of the form (state S: Dv x Dk, per chunk of
// C tokens with entry state S0)
//   A  = strictLower(diag(rs) Y X^T)          chunk Gram (read keys Y, write keys X)
//   T  = (I + A)^-1
//   W  = T diag(rs) (Z - Y S0^T)              row t of W is the token-t write
//   O  = Q S0^T + (Q X^T masked to i <= t) W  inclusive readout
//   S1 = S0 diag(g) + W^T X'                  exit state (g: exit decay)
// OSDN ([OSDN-it] 2.1): Y = K, X = X' = K~ (the preconditioned keys: K~
// replaces K in the Gram matrix and the intra-chunk scores), Z = V,
// rs = beta, g = 1. This is the token recurrence
// S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t) k~_t^T rewritten exactly.
//
// Work decomposition: one workgroup (4 waves) per (batch, head, VT-wide value
// tile), walking the chunks in order; the VT x Dk state slice lives in fp32
// MFMA accumulators. Value tiles are independent given the keys, so the
// V-independent chunk quantities (A, T, Q X^T) are recomputed per tile rather
// than written to and re-read from HBM. The next chunk's inputs are fetched
// into registers while the current chunk computes.
//
// T = (I + A)^-1: 16x16 diagonal blocks by fp32 forward substitution (one
// lane per column), then recursive doubling, merging pairs of s x s inverses
// into 2s x 2s ones with T21 = -T22 A21 T11 on MFMA.
#include "device_common.hpp"
#include "launch.hpp"

namespace osdn {

template <int DK, int C, int VT, typename Tin>
struct WyCfg {
  static constexpr int NW = 4, NT = 256;
  static constexpr int PAD = sizeof(Tin) == 2 ? 8 : 4;
  static constexpr int LDK = DK + PAD;
  static constexpr int LDC = C + PAD;
  static constexpr int LDF = C + 4;
  static constexpr int LDY = 32 + PAD;
  static constexpr int TB = C / 16, VB = VT / 16, DB = DK / 16;
  static constexpr int VEC = 16 / sizeof(Tin);
  static constexpr size_t E = sizeof(Tin);
  static constexpr size_t oX = 0;
  static constexpr size_t oY = oX + (size_t)C * LDK * E;
  static constexpr size_t oQ = oY + (size_t)C * LDK * E;
  static constexpr size_t oXT = oQ + (size_t)C * LDK * E;
  static constexpr size_t oS = oXT + (size_t)DK * LDC * E;
  static constexpr size_t oZ = oS + (size_t)VT * LDK * E;
  static constexpr size_t oRS = oZ + (size_t)C * VT * E;
  static constexpr size_t oA = oRS + (size_t)C * 4;
  static constexpr size_t oAb = oA + (size_t)C * LDF * 4;
  static constexpr size_t oTb = oAb + (size_t)C * LDC * E;
  static constexpr size_t oTt = oTb + (size_t)C * LDC * E;
  static constexpr size_t oYs = oTt + (size_t)C * LDC * E;
  static constexpr size_t oP = oYs + (size_t)32 * LDY * E;
  static constexpr size_t oR = oP + (size_t)C * LDC * E;
  static constexpr size_t oW = oR + (size_t)VT * LDC * E;
  static constexpr size_t bytes = oW + (size_t)VT * LDC * E;
  static constexpr bool fits = bytes <= 163840;
  static constexpr int NS = (VB * DB + NW - 1) / NW;  // state tiles per wave
  static constexpr int NO = (TB * VB + NW - 1) / NW;  // output tiles per wave
  // 16-byte vectors per thread for a C x DK and a C x VT chunk
  static constexpr int NLK = (C * DK / VEC + NT - 1) / NT;
  static constexpr int NLV = (C * VT / VEC + NT - 1) / NT;
};

// Register-staged inputs of one OSDN chunk (prefetched one chunk ahead).
template <int DK, int C, int VT, typename Tin>
struct OsdnChunkRegs {
  using G = WyCfg<DK, C, VT, Tin>;
  uint4 k[G::NLK], kt[G::NLK], q[G::NLK], v[G::NLV];
  float beta;

  __device__ __forceinline__ void load(const Tin* __restrict__ kp,
                                       const Tin* __restrict__ ktp,
                                       const Tin* __restrict__ qp,
                                       const Tin* __restrict__ vp,
                                       const float* __restrict__ bp, size_t t0,
                                       int valid, int Dv, int v0) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < G::NLK; ++i) {
      const int e = tid + i * G::NT;
      const int rr = e / (DK / G::VEC), cc = (e % (DK / G::VEC)) * G::VEC;
      uint4 z = {0u, 0u, 0u, 0u};
      k[i] = z; kt[i] = z; q[i] = z;
      if (e < C * DK / G::VEC && rr < valid) {
        const size_t g = (t0 + rr) * DK + cc;
        k[i] = *reinterpret_cast<const uint4*>(kp + g);
        kt[i] = *reinterpret_cast<const uint4*>(ktp + g);
        q[i] = *reinterpret_cast<const uint4*>(qp + g);
      }
    }
#pragma unroll
    for (int i = 0; i < G::NLV; ++i) {
      const int e = tid + i * G::NT;
      const int rr = e / (VT / G::VEC), cc = (e % (VT / G::VEC)) * G::VEC;
      uint4 z = {0u, 0u, 0u, 0u};
      v[i] = z;
      if (e < C * VT / G::VEC && rr < valid)
        v[i] = *reinterpret_cast<const uint4*>(vp + (t0 + rr) * Dv + v0 + cc);
    }
    beta = (tid < valid) ? bp[t0 + tid] : 0.f;
  }

  __device__ __forceinline__ void store(Tin* Xs, Tin* Ys, Tin* Qs, Tin* XTt,
                                        Tin* Zs, float* rs) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < G::NLK; ++i) {
      const int e = tid + i * G::NT;
      if (e < C * DK / G::VEC) {
        const int rr = e / (DK / G::VEC), cc = (e % (DK / G::VEC)) * G::VEC;
        *reinterpret_cast<uint4*>(Xs + rr * G::LDK + cc) = kt[i];
        *reinterpret_cast<uint4*>(Ys + rr * G::LDK + cc) = k[i];
        *reinterpret_cast<uint4*>(Qs + rr * G::LDK + cc) = q[i];
        const Tin* te = reinterpret_cast<const Tin*>(&kt[i]);
#pragma unroll
        for (int u = 0; u < G::VEC; ++u) XTt[(cc + u) * G::LDC + rr] = te[u];
      }
    }
#pragma unroll
    for (int i = 0; i < G::NLV; ++i) {
      const int e = tid + i * G::NT;
      if (e < C * VT / G::VEC) {
        const int rr = e / (VT / G::VEC), cc = (e % (VT / G::VEC)) * G::VEC;
        *reinterpret_cast<uint4*>(Zs + rr * VT + cc) = v[i];
      }
    }
    if (tid < C) rs[tid] = beta;
  }
};

template <int DK, int C, int VT, typename Tin>
__global__ __launch_bounds__(256) void osdn_wy_kernel(
    int T, int Dv, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ ktil, const Tin* __restrict__ v,
    const float* __restrict__ beta, const float* __restrict__ S0, float scale,
    Tin* __restrict__ o, float* __restrict__ ST) {
  using G = WyCfg<DK, C, VT, Tin>;
  constexpr int LDK = G::LDK, LDC = G::LDC, LDF = G::LDF, LDY = G::LDY;
  constexpr int TB = G::TB, VB = G::VB, DB = G::DB;
  __shared__ __attribute__((aligned(16))) unsigned char smem[G::bytes];
  Tin* Xs = reinterpret_cast<Tin*>(smem + G::oX);
  Tin* Ys = reinterpret_cast<Tin*>(smem + G::oY);
  Tin* Qs = reinterpret_cast<Tin*>(smem + G::oQ);
  Tin* XTt = reinterpret_cast<Tin*>(smem + G::oXT);
  Tin* Ss = reinterpret_cast<Tin*>(smem + G::oS);
  Tin* Zs = reinterpret_cast<Tin*>(smem + G::oZ);
  float* rs = reinterpret_cast<float*>(smem + G::oRS);
  float* Am = reinterpret_cast<float*>(smem + G::oA);
  Tin* Ab = reinterpret_cast<Tin*>(smem + G::oAb);
  Tin* Tb = reinterpret_cast<Tin*>(smem + G::oTb);
  Tin* Tt = reinterpret_cast<Tin*>(smem + G::oTt);
  Tin* Ysc = reinterpret_cast<Tin*>(smem + G::oYs);
  Tin* Pb = reinterpret_cast<Tin*>(smem + G::oP);
  Tin* Rt = reinterpret_cast<Tin*>(smem + G::oR);
  Tin* Wt = reinterpret_cast<Tin*>(smem + G::oW);

  const int nvt = Dv / VT;
  // XCD-aware numbering: workgroups go round-robin over the 8 XCDs; keep all
  // value tiles of one (batch, head) on one XCD so they share its L2.
  int lin = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) lin = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int bh = lin / nvt, vt = lin - bh * nvt;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int v0 = vt * VT;
  const size_t row0 = (size_t)bh * T;
  const Tin zero = from_f32<Tin>(0.f);

  // Blocks above the diagonal of T and P (below it for T^T) stay zero.
  for (int e = tid; e < C * C; e += G::NT) {
    const int rr = e / C, cc = e % C;
    if ((cc >> 4) > (rr >> 4)) {
      Tb[rr * LDC + cc] = zero;
      Pb[rr * LDC + cc] = zero;
      Tt[cc * LDC + rr] = zero;
    }
  }

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
  OsdnChunkRegs<DK, C, VT, Tin> regs;
  if (nchunks > 0) regs.load(k, ktil, q, v, beta, row0, min(C, T), Dv, v0);

  for (int j = 0; j < nchunks; ++j) {
    const size_t t0 = row0 + (size_t)j * C;
    const int valid = min(C, T - j * C);
    // ---- S1: operands of chunk j into LDS; prefetch chunk j+1 -------------
    regs.store(Xs, Ys, Qs, XTt, Zs, rs);
    if (j + 1 < nchunks)
      regs.load(k, ktil, q, v, beta, t0 + C, min(C, T - (j + 1) * C), Dv, v0);
    __syncthreads();

    // ---- S2: Gram A, scores P, RHS = rs (Z - Y S0^T), Q S0^T --------------
    constexpr int NL = TB * (TB + 1) / 2;
    for (int job = wave; job < 2 * NL + TB * VB; job += G::NW) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (job < 2 * NL) {
        const bool isP = job >= NL;
        int l = isP ? job - NL : job, a = 0;
        while (l > a) { l -= a + 1; ++a; }
        const int b = l;
        mma_nt<DK>(acc, (isP ? Qs : Ys) + a * 16 * LDK, LDK, Xs + b * 16 * LDK,
                   LDK);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = a * 16 + acc_row(i), cc = b * 16 + acc_col();
          if (isP) {
            Pb[rr * LDC + cc] = from_f32<Tin>(cc <= rr ? acc[i] : 0.f);
          } else {
            const float x = cc < rr ? rs[rr] * acc[i] : 0.f;
            Am[rr * LDF + cc] = x;
            Ab[rr * LDC + cc] = from_f32<Tin>(x);
          }
        }
      } else {
        const int l = job - 2 * NL, tb = l / VB, vb = l % VB;
        mma_nt<DK>(acc, Ys + tb * 16 * LDK, LDK, Ss + vb * 16 * LDK, LDK);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = tb * 16 + acc_row(i), cc = vb * 16 + acc_col();
          Rt[cc * LDC + rr] =
              from_f32<Tin>(rs[rr] * (to_f32(Zs[rr * VT + cc]) - acc[i]));
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

    // ---- S3: diagonal 16x16 blocks of T, fp32 forward substitution --------
    // Wave b < TB solves block b; lane c < 16 owns column c. Pending sums are
    // updated as soon as each entry is final, so the dependent chain is 15
    // FMAs long.
    if (wave < TB && lane < 16) {
      const int b = wave, c = lane;
      const float* Ablk = Am + b * 16 * LDF + b * 16;
      float x[16], s[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = (i == c) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        x[m] = s[m];
#pragma unroll
        for (int i = m + 1; i < 16; ++i) s[i] -= Ablk[i * LDF + m] * x[m];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const Tin xv = from_f32<Tin>(x[i]);
        Tb[(b * 16 + i) * LDC + b * 16 + c] = xv;
        Tt[(b * 16 + c) * LDC + b * 16 + i] = xv;
      }
    }
    __syncthreads();

    // ---- S4: recursive doubling, T21 = -T22 (A21 T11) ----------------------
#pragma unroll
    for (int s = 16; s < C; s *= 2) {
      const int npair = C / (2 * s);
      const int nt = s / 16;                 // tiles per side of an s x s block
      const int jobs = npair * nt * nt;
      // Y = A21 T11 (s x s, K = s), stored transposed in the scratch.
      for (int job = wave; job < jobs; job += G::NW) {
        const int p = job / (nt * nt), r = (job / nt) % nt, c = job % nt;
        const int rb = 2 * s * p + s, cb = 2 * s * p;   // A21 origin
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < s; kk += 16)
          mma_nt<16>(acc, Ab + (rb + r * 16) * LDC + cb + kk, LDC,
                     Tt + (cb + c * 16) * LDC + cb + kk, LDC);
        Tin* ys = Ysc + (p * s) * LDY;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ys[(c * 16 + acc_col()) * LDY + r * 16 + acc_row(i)] = from_f32<Tin>(acc[i]);
      }
      __syncthreads();
      // T21 = -T22 Y
      for (int job = wave; job < jobs; job += G::NW) {
        const int p = job / (nt * nt), r = (job / nt) % nt, c = job % nt;
        const int rb = 2 * s * p + s, cb = 2 * s * p;
        const Tin* ys = Ysc + (p * s) * LDY;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < s; kk += 16)
          mma_nt<16>(acc, Tb + (rb + r * 16) * LDC + rb + kk, LDC,
                     ys + (c * 16) * LDY + kk, LDY);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = rb + r * 16 + acc_row(i), cc = cb + c * 16 + acc_col();
          const Tin xv = from_f32<Tin>(-acc[i]);
          Tb[rr * LDC + cc] = xv;
          Tt[cc * LDC + rr] = xv;
        }
      }
      __syncthreads();
    }

    // ---- S5: W = T RHS, stored transposed ---------------------------------
    for (int job = wave; job < TB * VB; job += G::NW) {
      const int tb = job / VB, vb = job % VB;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mma_nt<C>(acc, Tb + tb * 16 * LDC, LDC, Rt + vb * 16 * LDC, LDC);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Wt[(vb * 16 + acc_col()) * LDC + tb * 16 + acc_row(i)] = from_f32<Tin>(acc[i]);
    }
    __syncthreads();

    // ---- S6: O += P W (store), S += W^T X ----------------------------------
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
        mma_nt<C>(Sacc[s], Wt + vb * 16 * LDC, LDC, XTt + db * 16 * LDC, LDC);
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
  if constexpr (!WyCfg<DK, C, VT, Tin>::fits) {
    return -1;
  } else {
    const int BH = a.B * a.H;
    dim3 grid(BH * (a.Dv / VT)), block(256);
    hipLaunchKernelGGL((osdn_wy_kernel<DK, C, VT, Tin>), grid, block, 0, s,
                       a.T, a.Dv, (const Tin*)a.q, (const Tin*)a.k,
                       (const Tin*)a.ktilde, (const Tin*)a.v, a.beta, a.S0,
                       a.scale, (Tin*)a.o, a.ST);
    return (int)hipGetLastError();
  }
}

// Value-tile width: 32 columns when that already gives one workgroup per
// compute unit (256 CUs), else 16 for more parallelism.
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
  switch (chunk) {
    case 16: return WyCfg<DK, 16, 32, Tin>::fits && WyCfg<DK, 16, 16, Tin>::fits;
    case 32: return WyCfg<DK, 32, 32, Tin>::fits && WyCfg<DK, 32, 16, Tin>::fits;
    case 64: return WyCfg<DK, 64, 32, Tin>::fits && WyCfg<DK, 64, 16, Tin>::fits;
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
