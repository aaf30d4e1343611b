// Phase 1 of the OSDN forward: the preconditioner scan over the key stream,
// in chunked form.
//
// [OSDN-it] sections 2.2 and 2.3 define, per (batch, head) and token t,
//   a_t = k_t*k_t, n_t = ||k_t||^2, c_t = <d_t, a_t>, k~_t = d_t * k_t,
//   g_t = eta beta_t (1 - beta_t c_t) / n_t          (0 when n_t = 0),
//   d_{t+1} = r_t d_t + g_t a_t                       (descent on the closed-form
//                                                     surrogate, gate r_t).
// The step is affine in d, so a chunk of C tokens with entry value d0 is
// solved at once. With P_t = prod_{j<t} r_j (P_0 = 1) inside the chunk,
//   d_t   = P_t d0 + sum_{i<t} (P_t / P_{i+1}) g_i a_i,
//   c_t   = P_t <d0, a_t> + sum_{i<t} (P_t / P_{i+1}) g_i <a_i, a_t>,
// so g solves the unit lower-triangular system (I + M) g = b with
//   M[t][i] = (eta beta_t^2 / n_t) (P_t / P_{i+1}) <a_i, a_t>   (i < t),
//   b_t     = (eta beta_t / n_t) (1 - beta_t P_t <d0, a_t>).
// M depends on the keys and gates only, so the Gram matrix and the inverse
// (I + M)^-1 are computed without d; the serial part per chunk is three
// matrix-vector products (<d0, a_t>, the inverse applied to b, and the exit
// value d_C). The preconditioned keys of the chunk follow as
// K~ = (P d0^T + L A) * K with L[t][i] = (P_t / P_{i+1}) g_i for i < t.
//
// One workgroup (4 waves) per (batch, head) walks the chunks in order.
// Precision: d never passes through bf16. The Gram matrix of a is formed on
// MFMA from an exact two-term bf16 split of a (a bf16 key squared has a 16-bit
// significand), the inverse and the chain run in fp32; only the correction
// term L A of K~, rounded afterwards to the key dtype, uses bf16 operands.
#include "device_common.hpp"
#include "launch.hpp"

namespace osdn {

template <int DK, int C, typename Tin>
struct PcCfg {
  static constexpr int NW = 4, NT = 256;
  static constexpr int PAD = sizeof(Tin) == 2 ? 8 : 4;
  static constexpr int LDK = DK + PAD;      // rows of Dk key elements
  static constexpr int LDH = DK + 8;        // rows of Dk bf16 elements
  static constexpr int LDC = C + PAD;       // rows of C operand elements
  static constexpr int LDF = C + 4;         // rows of C fp32 elements
  static constexpr int LDY = 32 + 4;        // fp32 merge scratch
  static constexpr int TB = C / 16, DB = DK / 16;
  static constexpr int VEC = 16 / sizeof(Tin);
  static constexpr int NCB = DK / VEC;      // 16-byte column blocks per key row
  static constexpr int NLK = (C * NCB + NT - 1) / NT;
  static constexpr size_t E = sizeof(Tin);
  static constexpr size_t oK = 0;
  static constexpr size_t oAh = oK + (size_t)C * LDK * E;
  static constexpr size_t oAl = oAh + (size_t)C * LDH * 2;
  static constexpr size_t oAT = oAl + (size_t)C * LDH * 2;
  static constexpr size_t oM = oAT + (size_t)DK * LDC * E;
  static constexpr size_t oT = oM + (size_t)C * LDF * 4;
  static constexpr size_t oTt = oT + (size_t)C * LDF * 4;
  static constexpr size_t oY = oTt + (size_t)C * LDF * 4;
  static constexpr size_t oL = oY + (size_t)32 * LDY * 4;
  static constexpr size_t oV = oL + (size_t)C * LDC * E;
  // vectors: n, beta, rho, e, lp (C+4), P (C+4), lambda, b, g (C each);
  // d0, dn (DK each); per-thread partial norms (NT)
  static constexpr size_t bytes = oV + (size_t)(9 * C + 8 + 2 * DK + NT) * 4;
  static constexpr bool fits = bytes <= 163840;
  // The K~ staging buffer reuses the (no longer needed) split-a buffers.
  static_assert((size_t)C * LDK * E <= (size_t)2 * C * LDH * 2, "staging");
};

template <typename Tin>
__device__ __forceinline__ void split_bf16(float a, __bf16& hi, __bf16& lo) {
  hi = (__bf16)a;
  lo = (__bf16)(a - (float)hi);
}

template <int DK, int C, typename Tin>
__global__ __launch_bounds__(256) void precond_chunk_kernel(
    int T, const Tin* __restrict__ k, const float* __restrict__ beta,
    const float* __restrict__ r, float eta, const float* __restrict__ d0in,
    Tin* __restrict__ ktil, float* __restrict__ dT) {
  using G = PcCfg<DK, C, Tin>;
  constexpr int LDK = G::LDK, LDH = G::LDH, LDC = G::LDC, LDF = G::LDF,
                LDY = G::LDY, TB = G::TB, DB = G::DB, VEC = G::VEC;
  __shared__ __attribute__((aligned(16))) unsigned char smem[G::bytes];
  Tin* Ks = reinterpret_cast<Tin*>(smem + G::oK);
  __bf16* Ah = reinterpret_cast<__bf16*>(smem + G::oAh);
  __bf16* Al = reinterpret_cast<__bf16*>(smem + G::oAl);
  Tin* KTst = reinterpret_cast<Tin*>(smem + G::oAh);   // aliases Ah, Al
  Tin* ATt = reinterpret_cast<Tin*>(smem + G::oAT);
  float* Mf = reinterpret_cast<float*>(smem + G::oM);
  float* Tf = reinterpret_cast<float*>(smem + G::oT);
  float* Tft = reinterpret_cast<float*>(smem + G::oTt);
  float* Ysc = reinterpret_cast<float*>(smem + G::oY);
  Tin* Lb = reinterpret_cast<Tin*>(smem + G::oL);
  float* nv = reinterpret_cast<float*>(smem + G::oV);
  float* bev = nv + C;           // beta
  float* rhov = bev + C;         // eta beta^2 / n
  float* ev = rhov + C;          // eta beta / n
  float* lpv = ev + C;           // C + 4 slots: lp[0..C], lp_t = sum_{j<t} log r_j
  float* Pv = lpv + C + 4;       // C + 4 slots: P_t = exp(lp_t)
  float* lamv = Pv + C + 4;      // P_C / P_{i+1}
  float* bvec = lamv + C;
  float* gv = bvec + C;
  float* d0v = gv + C;
  float* dnv = d0v + DK;
  float* npart = dnv + DK;       // NT partial key norms

  const int bh = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int NCB = G::NCB;
  const size_t row0 = (size_t)bh * T;
  const float* bp = beta + row0;
  const float* rp = r ? r + row0 : nullptr;

  for (int c = tid; c < DK; c += G::NT)
    d0v[c] = d0in ? d0in[(size_t)bh * DK + c] : 1.f;
  // Upper 16x16 blocks of the inverse (and its transpose's lower blocks)
  // and of L stay zero.
  for (int e = tid; e < C * C; e += G::NT) {
    const int rr = e / C, cc = e % C;
    if ((cc >> 4) > (rr >> 4)) {
      Tf[rr * LDF + cc] = 0.f;
      Tft[cc * LDF + rr] = 0.f;
    }
    if (cc >= rr) Lb[rr * LDC + cc] = from_f32<Tin>(0.f);
  }

  const int nchunks = (T + C - 1) / C;
  uint4 kr[G::NLK];
  float br = 0.f, rr_ = 1.f;
  auto prefetch = [&](int j) {
    const int valid = min(C, T - j * C);
    const size_t t0 = row0 + (size_t)j * C;
#pragma unroll
    for (int i = 0; i < G::NLK; ++i) {
      const int e = tid + i * G::NT;
      const int rr = e % C, cc = (e / C) * VEC;
      kr[i] = uint4{0u, 0u, 0u, 0u};
      if (e < C * NCB && rr < valid)
        kr[i] = *reinterpret_cast<const uint4*>(k + (t0 + rr) * DK + cc);
    }
    br = (tid < valid) ? bp[(size_t)j * C + tid] : 0.f;
    rr_ = (tid < valid && rp) ? rp[(size_t)j * C + tid] : 1.f;
  };
  if (nchunks > 0) prefetch(0);

  for (int j = 0; j < nchunks; ++j) {
    const int valid = min(C, T - j * C);
    const size_t t0 = row0 + (size_t)j * C;
    // ---- A: keys, squares (split), transposed squares, norms, gates ------
    // Each lane owns one token row, so the transposed writes of a from
    // consecutive lanes land in consecutive LDS addresses.
    {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < G::NLK; ++i) {
        const int e = tid + i * G::NT;
        if (e < C * NCB) {
          const int rr = e % C, cc = (e / C) * VEC;
          *reinterpret_cast<uint4*>(Ks + rr * LDK + cc) = kr[i];
          const Tin* kv = reinterpret_cast<const Tin*>(&kr[i]);
          __bf16 hi[VEC], lo[VEC];
#pragma unroll
          for (int u = 0; u < VEC; ++u) {
            const float x = to_f32(kv[u]);
            const float a = x * x;
            part += a;
            split_bf16<Tin>(a, hi[u], lo[u]);
            ATt[(cc + u) * LDC + rr] = from_f32<Tin>(a);
          }
          if constexpr (VEC == 8) {
            *reinterpret_cast<uint4*>(Ah + rr * LDH + cc) = *reinterpret_cast<const uint4*>(hi);
            *reinterpret_cast<uint4*>(Al + rr * LDH + cc) = *reinterpret_cast<const uint4*>(lo);
          } else {
            *reinterpret_cast<uint2*>(Ah + rr * LDH + cc) = *reinterpret_cast<const uint2*>(hi);
            *reinterpret_cast<uint2*>(Al + rr * LDH + cc) = *reinterpret_cast<const uint2*>(lo);
          }
        }
      }
      npart[tid] = part;   // row tid % C, summed over this thread's blocks
    }
    if (wave == 0) {
      // exclusive prefix of log r over the chunk (r clamped away from 0 so
      // that ratios of prefixes stay finite)
      const float lr = (lane < C) ? logf(fmaxf(rr_, 1e-30f)) : 0.f;
      const float inc = wave_prefix_sum(lr);
      if (lane < C) {
        lpv[lane] = inc - lr;
        bev[lane] = br;
      }
      if (lane == C - 1) lpv[C] = inc;
    }
    if (j + 1 < nchunks) prefetch(j + 1);
    __syncthreads();

    // ---- B: per-token scalars; Gram of a (split bf16 MFMA) ------------------
    if (wave == 0 && lane < C) {
      const int t = lane;
      float n = 0.f;
#pragma unroll
      for (int m = 0; m < G::NT / C; ++m) n += npart[t + m * C];
      const float bt = bev[t];
      nv[t] = n;
      ev[t] = n > 0.f ? eta * bt / n : 0.f;
      rhov[t] = n > 0.f ? eta * bt * bt / n : 0.f;
      Pv[t] = expf(lpv[t]);
      lamv[t] = expf(lpv[C] - lpv[t + 1]);
      if (t == C - 1) Pv[C] = expf(lpv[C]);
    }
    // Tile list: wave w owns the diagonal tile (w, w) and a share of the
    // off-diagonal lower tiles, and keeps its accumulators in registers.
    constexpr int NL = TB * (TB + 1) / 2;
    constexpr int NJ = 1 + (NL - TB + G::NW - 1) / G::NW;
    f32x4 gacc[NJ];
    int gja[NJ], gjb[NJ];
#pragma unroll
    for (int s2 = 0; s2 < NJ; ++s2) {
      int a = -1, b = -1;
      const int job = wave + G::NW * s2;
      if (s2 == 0) {
        if (wave < TB) { a = wave; b = wave; }
      } else {
        // off-diagonal tiles in row-major order, dealt round-robin
        int l = job - G::NW, aa = 1;
        if (l >= 0) {
          while (l >= aa) { l -= aa; ++aa; }
          if (aa < TB) { a = aa; b = l; }
        }
      }
      gja[s2] = a;
      gjb[s2] = b;
      gacc[s2] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (a >= 0) {
        mma_nt<DK>(gacc[s2], Ah + a * 16 * LDH, LDH, Ah + b * 16 * LDH, LDH);
        mma_nt<DK>(gacc[s2], Ah + a * 16 * LDH, LDH, Al + b * 16 * LDH, LDH);
        mma_nt<DK>(gacc[s2], Al + a * 16 * LDH, LDH, Ah + b * 16 * LDH, LDH);
      }
    }
    __syncthreads();
    // M[t][i] = rho_t (P_t / P_{i+1}) <a_i, a_t> for i < t
#pragma unroll
    for (int s2 = 0; s2 < NJ; ++s2) {
      const int a = gja[s2], b = gjb[s2];
      if (a >= 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = a * 16 + acc_row(i), c = b * 16 + acc_col();
          Mf[t * LDF + c] =
              c < t ? rhov[t] * __expf(lpv[t] - lpv[c + 1]) * gacc[s2][i] : 0.f;
        }
      }
    }

    // ---- C: diagonal 16x16 blocks of (I + M)^-1 ----------------------------
    // Wave b wrote diagonal tile (b, b) of M itself, so it can invert it
    // without waiting for the other waves.
    if (wave < TB && lane < 16) {
      const int b = wave, c = lane;
      const float* Mblk = Mf + b * 16 * LDF + b * 16;
      float x[16], s[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = (i == c) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        x[m] = s[m];
#pragma unroll
        for (int i = m + 1; i < 16; ++i) s[i] -= Mblk[i * LDF + m] * x[m];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        Tf[(b * 16 + i) * LDF + b * 16 + c] = x[i];
        Tft[(b * 16 + c) * LDF + b * 16 + i] = x[i];
      }
    }
    __syncthreads();

    // ---- D: recursive doubling in fp32, T21 = -T22 (M21 T11) ---------------
#pragma unroll
    for (int s = 16; s < C; s *= 2) {
      const int npair = C / (2 * s), nt = s / 16, jobs = npair * nt * nt;
      for (int job = wave; job < jobs; job += G::NW) {
        const int p = job / (nt * nt), rt = (job / nt) % nt, ct = job % nt;
        const int rb = 2 * s * p + s, cb = 2 * s * p;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < s; kk += 16)
          mma_nt<16>(acc, Mf + (rb + rt * 16) * LDF + cb + kk, LDF,
                     Tft + (cb + ct * 16) * LDF + cb + kk, LDF);
        float* ys = Ysc + (p * s) * LDY;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ys[(ct * 16 + acc_col()) * LDY + rt * 16 + acc_row(i)] = acc[i];
      }
      __syncthreads();
      for (int job = wave; job < jobs; job += G::NW) {
        const int p = job / (nt * nt), rt = (job / nt) % nt, ct = job % nt;
        const int rb = 2 * s * p + s, cb = 2 * s * p;
        const float* ys = Ysc + (p * s) * LDY;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < s; kk += 16)
          mma_nt<16>(acc, Tf + (rb + rt * 16) * LDF + rb + kk, LDF,
                     ys + (ct * 16) * LDY + kk, LDY);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = rb + rt * 16 + acc_row(i), cc = cb + ct * 16 + acc_col();
          Tf[rr * LDF + cc] = -acc[i];
          Tft[cc * LDF + rr] = -acc[i];
        }
      }
      __syncthreads();
    }

    // ---- E: the serial chain --------------------------------------------------
    // p_t = <d0, a_t>; b_t = (eta beta_t / n_t)(1 - beta_t P_t p_t)
    {
      constexpr int Q = 256 / C;            // threads per token row
      constexpr int SEG = DK / Q;           // contiguous channels per thread
      const int t = tid / Q, q = tid % Q;
      const Tin* krow = Ks + t * LDK + q * SEG;
      const float* drow = d0v + q * SEG;
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < SEG; ++c) {
        const float x = to_f32(krow[c]);
        s += x * x * drow[c];
      }
      s = group_sum<Q>(s);
      if (q == 0) bvec[t] = ev[t] * (1.f - bev[t] * Pv[t] * s);
    }
    __syncthreads();
    // g = (I + M)^-1 b (the inverse is zero above the diagonal)
    {
      constexpr int Q = 256 / C;
      constexpr int SEG = C / Q;
      const int t = tid / Q, q = tid % Q;
      const float* trow = Tf + t * LDF + q * SEG;
      const float* bseg = bvec + q * SEG;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < SEG; ++i) s += trow[i] * bseg[i];
      s = group_sum<Q>(s);
      if (q == 0) gv[t] = s;
    }
    __syncthreads();
    // exit value d_C = P_C d0 + sum_i (P_C / P_{i+1}) g_i a_i, and L
    {
      constexpr int Q = 256 / DK;           // threads per channel (2, 4 or 8)
      const int c = tid / Q, q = tid % Q;
      float s = 0.f;
      for (int i = q; i < C; i += Q) {
        const float x = to_f32(Ks[i * LDK + c]);
        s += lamv[i] * gv[i] * x * x;
      }
      s = group_sum<Q>(s);
      if (q == 0) dnv[c] = Pv[C] * d0v[c] + s;
      for (int e = tid; e < C * C; e += G::NT) {
        const int t = e / C, i = e % C;
        if (i < t) Lb[t * LDC + i] = from_f32<Tin>(__expf(lpv[t] - lpv[i + 1]) * gv[i]);
      }
    }
    __syncthreads();

    // ---- F: K~ = (P d0^T + L A) * K, staged in LDS, stored coalesced --------
    for (int job = wave; job < TB * DB; job += G::NW) {
      const int tb = job / DB, db = job % DB;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mma_nt<C>(acc, Lb + tb * 16 * LDC, LDC, ATt + db * 16 * LDC, LDC);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tb * 16 + acc_row(i), c = db * 16 + acc_col();
        const float dt = Pv[t] * d0v[c] + acc[i];
        KTst[t * LDK + c] = from_f32<Tin>(dt * to_f32(Ks[t * LDK + c]));
      }
    }
    __syncthreads();
    if (ktil) {
#pragma unroll
      for (int i = 0; i < G::NLK; ++i) {
        const int e = tid + i * G::NT;
        const int rr = e / NCB, cc = (e % NCB) * VEC;
        if (e < C * NCB && rr < valid)
          *reinterpret_cast<uint4*>(ktil + (t0 + rr) * DK + cc) =
              *reinterpret_cast<const uint4*>(KTst + rr * LDK + cc);
      }
    }
    for (int c = tid; c < DK; c += G::NT) d0v[c] = dnv[c];
    __syncthreads();
  }
  if (dT)
    for (int c = tid; c < DK; c += G::NT) dT[(size_t)bh * DK + c] = d0v[c];
}

template <int DK, typename Tin>
static int launch_dk(const PrecondArgs& a, hipStream_t s) {
  // Phase-1 chunk: 64 tokens for bf16 keys, 32 for fp32 keys (LDS budget).
  constexpr int C = sizeof(Tin) == 2 ? 64 : 32;
  static_assert(PcCfg<DK, C, Tin>::fits, "phase-1 working set exceeds LDS");
  dim3 grid(a.B * a.H), block(256);
  hipLaunchKernelGGL((precond_chunk_kernel<DK, C, Tin>), grid, block, 0, s,
                     a.T, (const Tin*)a.k, a.beta, a.r, a.eta, a.d0,
                     (Tin*)a.ktilde, a.dT);
  return (int)hipGetLastError();
}

int launch_precond_scan(const PrecondArgs& a, hipStream_t s) {
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

}  // namespace osdn
