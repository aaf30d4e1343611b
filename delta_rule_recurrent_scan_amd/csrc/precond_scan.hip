// Phase 1 of the OSDN forward: the preconditioner scan over the key stream,
// in chunk-parallel form.
//
// [OSDN-it] sections 2.2 and 2.3 define, per (batch, head) and token t,
//   a_t = k_t*k_t, n_t = ||k_t||^2, x_t = <d_t, a_t>, k~_t = d_t * k_t,
//   g_t = eta beta_t (1 - beta_t x_t) / n_t          (0 when n_t = 0),
//   d_{t+1} = r_t d_t + g_t a_t                       (descent on the closed-form
//                                                     surrogate, gate r_t).
// The step is affine in d, so a chunk of C tokens with entry value d0 is
// solved at once. With P_t = prod_{j<t} r_j (P_0 = 1) inside the chunk,
//   d_t   = P_t d0 + sum_{i<t} (P_t / P_{i+1}) g_i a_i,
// and g solves the unit lower-triangular system (I + M) g = b with
//   M[t][i] = (eta beta_t^2 / n_t) (P_t / P_{i+1}) <a_i, a_t>   (i < t),
//   b_t     = e_t - h_t <d0, a_t>,  e_t = eta beta_t / n_t,  h_t = e_t beta_t P_t.
// With T = (I + M)^-1, g0 = T e and V = T diag(h), and x = A d0 (rows a_t):
//   g   = g0 - V x,
//   d_C = P_C d0 + A^T (c * g),   c_i = P_C / P_{i+1},
//   K~  = (P d0^T + L A) * K,     L[t][i] = (P_t / P_{i+1}) g_i  (i < t).
// Only the middle line links the chunks. Three kernels:
//   prep    persistent workgroups over all chunks at once (the next chunk
//           fetched during the current one): the Gram matrix of a, M, T,
//           and the chunk record {log P prefix, g0, V};
//   chain   one workgroup per (batch, head): the serial part, three
//           matrix-vector products per chunk (x = A d, g = g0 - V x,
//           d <- P_C d + A^T (c*g)); records d at each chunk entry and g;
//   ktilde  one workgroup per chunk: K~ from d, g and the keys.
// Precision: d never passes through bf16. The Gram matrix of a is formed on
// MFMA from an exact two-term bf16 split of a (a bf16 key squared has a 16-bit
// significand), T and V are fp32 and the chain runs in fp32; only the ktilde
// kernel's correction term L A (chunks of 16 and 32 tokens), rounded
// afterwards to the key dtype, uses operands in the key dtype (at chunk 64
// the phase-2 prep forms K~ from d's own recursion in fp32).
#include "device_common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace osdn {

template <int DK, typename Tin>
struct P1Cfg {
  static constexpr int C = kPrecondChunk, NW = 4, NT = 256, TB = C / 16,
                       DB = DK / 16;
  static_assert(C == 64, "one token per lane in the gate prefix");
  static constexpr size_t E = sizeof(Tin);
  static constexpr int VEC = 16 / sizeof(Tin);
  static constexpr int NCB = DK / VEC;           // 16-byte blocks per key row
  static constexpr int NLK = C * NCB / NT;       // key blocks per thread
  static_assert((C * NCB) % NT == 0, "whole key blocks per thread");
  // chunk record (fp32): lp_0..lp_C (lp_t = log P_t), g (g0 from prep,
  // replaced by g in the chain), V (C x C, zero above the diagonal)
  static constexpr int R_LP = kRecLp, R_G = kRecG, R_V = kRecV, R_CF = kRecCf,
                       R_PC = kRecPc;
  static constexpr int RS = kRecStride;
  // prep: split squares (bf16), then T and the doubling scratch in their place
  static constexpr int LDH = DK + 8;
  static constexpr int LDF = C + 4;
  static constexpr int LDYS = 16 + 4;
  // shared Y of the widest doubling level (C/2 x C/2), rows 16 banks apart
  // for the k-major reads
  static constexpr int LDY = C / 2 + 16;
  static constexpr size_t uY = (size_t)NW * (C / 2) * LDYS * 4 > (size_t)(C / 2) * LDY * 4
                                   ? (size_t)NW * (C / 2) * LDYS * 4
                                   : (size_t)(C / 2) * LDY * 4;
  static constexpr size_t uSplit = (size_t)2 * C * LDH * 2;
  static constexpr size_t uT = (size_t)C * LDF * 4 + uY;
  static constexpr size_t pAh = 0, pAl = (size_t)C * LDH * 2;
  static constexpr size_t pT = 0, pY = (size_t)C * LDF * 4;
  static constexpr size_t pM = uSplit > uT ? uSplit : uT;
  static constexpr size_t pVec = pM + (size_t)C * LDF * 4;
  static constexpr size_t prep_bytes = pVec + (size_t)(C + 4 + 5 * C) * 4;
  // ktilde: keys (overwritten in place by K~), squares, L
  static constexpr int PAD = sizeof(Tin) == 2 ? 8 : 4;
  static constexpr int LDK = DK + PAD, LDC = C + PAD;
  static constexpr size_t kK = 0, kA = kK + (size_t)C * LDK * E;
  static constexpr size_t kL = kA + (size_t)C * LDK * E;
  static constexpr size_t kVec = kL + (size_t)C * LDC * E;
  static constexpr size_t kt_bytes = kVec + (size_t)(C + 4 + 2 * C + DK) * 4;
  static_assert(prep_bytes <= 163840 && kt_bytes <= 163840, "LDS");
};

__device__ __forceinline__ void split_bf16(float a, __bf16& hi, __bf16& lo) {
  hi = (__bf16)a;
  lo = (__bf16)(a - (float)hi);
}

// ---------------------------------------------------------------------------
// prep: everything of a chunk that does not depend on d
// ---------------------------------------------------------------------------
// Persistent: workgroup g takes chunks g, g + gridDim.x, ... and fetches the
// next chunk's keys and gates while the current one computes.
template <int DK, typename Tin>
__global__ __launch_bounds__(256) void precond_prep_kernel(
    int T, int nchunks, int total, const Tin* __restrict__ k,
    const float* __restrict__ beta, const float* __restrict__ r, float eta,
    float* __restrict__ rec) {
  using G = P1Cfg<DK, Tin>;
  constexpr int C = G::C, LDH = G::LDH, LDF = G::LDF, LDYS = G::LDYS,
                TB = G::TB, VEC = G::VEC, NCB = G::NCB;
  __shared__ __attribute__((aligned(16))) unsigned char smem[G::prep_bytes];
  __bf16* Ah = reinterpret_cast<__bf16*>(smem + G::pAh);
  __bf16* Al = reinterpret_cast<__bf16*>(smem + G::pAl);
  float* Tf = reinterpret_cast<float*>(smem + G::pT);     // after the Gram
  float* Ysc = reinterpret_cast<float*>(smem + G::pY);    // after the Gram
  float* Mf = reinterpret_cast<float*>(smem + G::pM);
  float* lpv = reinterpret_cast<float*>(smem + G::pVec);  // C + 4
  float* bev = lpv + C + 4;
  float* nv = bev + C;
  float* ev = nv + C;     // eta beta / n
  float* rho = ev + C;    // eta beta^2 / n
  float* hv = rho + C;    // rho P
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;

  // next chunk's keys (row e / NCB, 16-byte block e % NCB) and, on wave 0,
  // its gates (token = lane); padding tokens read as zero keys, r = 1, beta = 0
  uint4 kr[G::NLK];
  float rt = 1.f, bt = 0.f;
  auto fetch = [&](int n) {
    const int bh = n / nchunks, j = n - bh * nchunks;
    const int valid = min(C, T - j * C);
    const size_t t0 = (size_t)bh * T + (size_t)j * C;
#pragma unroll
    for (int i = 0; i < G::NLK; ++i) {
      const int e = tid + i * G::NT;
      const int rr = e / NCB, cc = (e % NCB) * VEC;
      kr[i] = uint4{0u, 0u, 0u, 0u};
      if (rr < valid) kr[i] = *reinterpret_cast<const uint4*>(k + (t0 + rr) * DK + cc);
    }
    if (wave == 0) {
      rt = (lane < valid && r) ? r[t0 + lane] : 1.f;
      bt = (lane < valid) ? beta[t0 + lane] : 0.f;
    }
  };
  if ((int)blockIdx.x < total) fetch(blockIdx.x);

  for (int n = blockIdx.x; n < total; n += gridDim.x) {
    float* out = rec + (size_t)n * G::RS;

    // ---- keys: split squares and row norms; gates --------------------------
#pragma unroll
    for (int i = 0; i < G::NLK; ++i) {
      const int e = tid + i * G::NT;
      const int rr = e / NCB, cc = (e % NCB) * VEC;
      const Tin* kv = reinterpret_cast<const Tin*>(&kr[i]);
      __bf16 hi[VEC], lo[VEC];
      float part = 0.f;
#pragma unroll
      for (int u = 0; u < VEC; ++u) {
        const float x = to_f32(kv[u]);
        const float a = x * x;
        part += a;
        split_bf16(a, hi[u], lo[u]);
      }
      if constexpr (VEC == 8) {
        *reinterpret_cast<uint4*>(Ah + rr * LDH + cc) = *reinterpret_cast<const uint4*>(hi);
        *reinterpret_cast<uint4*>(Al + rr * LDH + cc) = *reinterpret_cast<const uint4*>(lo);
      } else {
        *reinterpret_cast<uint2*>(Ah + rr * LDH + cc) = *reinterpret_cast<const uint2*>(hi);
        *reinterpret_cast<uint2*>(Al + rr * LDH + cc) = *reinterpret_cast<const uint2*>(lo);
      }
      // the NCB lanes of one row are consecutive and aligned
      part = group_sum<NCB>(part);
      if (e % NCB == 0) nv[rr] = part;
    }
    if (wave == 0) {
      // exclusive prefix of log r (r clamped away from 0 so that ratios of
      // prefixes stay finite)
      const float lr = logf(fmaxf(rt, 1e-30f));
      const float inc = wave_prefix_sum(lr);
      lpv[lane] = inc - lr;
      if (lane == C - 1) lpv[C] = inc;
      bev[lane] = bt;
    }
    if (n + (int)gridDim.x < total) fetch(n + gridDim.x);
    __syncthreads();

    // ---- per-token scalars; Gram of a (split bf16 MFMA) ----------------------
    if (wave == 0) {
      const int t = lane;
      const float n = nv[t], bt = bev[t];
      const float e = n > 0.f ? eta * bt / n : 0.f;
      ev[t] = e;
      rho[t] = e * bt;
      hv[t] = e * bt * expf(lpv[t]);
    }
    // Gram tiles (row block a >= column block b), dealt so that wave w < 2
    // owns those of diagonal pair w, (2w, 2w), (2w+1, 2w+1) and (2w+1, 2w),
    // and can invert the pair by itself; waves 2 and 3 own (w, 0) and (w, 1),
    // the tiles the second doubling level reads. Accumulators stay in
    // registers.
    static_assert(TB == 4 && G::NW == 4, "four 16-token blocks, four waves");
    constexpr int NJ = 3;
    f32x4 gacc[NJ];
    int gja[NJ], gjb[NJ];
#pragma unroll
    for (int s2 = 0; s2 < NJ; ++s2) {
      int a = -1, b = -1;
      if (wave < 2) {
        a = 2 * wave + (s2 >= 1);
        b = 2 * wave + (s2 == 1);
      } else if (s2 < 2) {
        a = wave;
        b = s2;
      }
      gja[s2] = a;
      gjb[s2] = b;
      gacc[s2] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (a >= 0) {
        Frag<DK, __bf16> ah, al, bh_, bl;
        ah.load(Ah + a * 16 * LDH, LDH);
        al.load(Al + a * 16 * LDH, LDH);
        bh_.load(Ah + b * 16 * LDH, LDH);
        bl.load(Al + b * 16 * LDH, LDH);
        // tile (b, a) of the symmetric Gram, so that a lane holds four
        // consecutive columns of one row of tile (a, b)
        mma(gacc[s2], bh_, ah);
        mma(gacc[s2], bl, ah);
        mma(gacc[s2], bh_, al);
      }
    }
    __syncthreads();  // the split squares are dead from here on (T reuses them)
    // M[t][i] = rho_t (P_t / P_{i+1}) <a_i, a_t> for i < t
#pragma unroll
    for (int s2 = 0; s2 < NJ; ++s2) {
      const int a = gja[s2], b = gjb[s2];
      if (a >= 0) {
        const int t = a * 16 + acc_col(), c0 = b * 16 + acc_row(0);
        float mv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = c0 + i;
          mv[i] = c < t ? rho[t] * __expf(lpv[t] - lpv[c + 1]) * gacc[s2][i] : 0.f;
        }
        *reinterpret_cast<float4*>(Mf + t * LDF + c0) = float4{mv[0], mv[1], mv[2], mv[3]};
      }
    }
    // Blocks of T above the diagonal are zero (four entries per access).
    for (int e4 = tid; e4 < C * C / 4; e4 += G::NT) {
      const int rr = e4 / (C / 4), cc = (e4 % (C / 4)) * 4;
      if ((cc >> 4) > (rr >> 4))
        *reinterpret_cast<float4*>(Tf + rr * LDF + cc) = float4{0.f, 0.f, 0.f, 0.f};
    }

    if (wave < 2) {
      // ---- diagonal pair `wave` of T = (I + M)^-1, by this wave alone -------
      // 16x16 diagonal blocks by forward substitution: lanes 0-15 take block
      // 2w, lanes 16-31 block 2w + 1, lane c % 16 owns column c % 16.
      wave_lds_sync();
      if (lane < 32) {
        const int b = 2 * wave + (lane >> 4), c = lane & 15;
        const float* Mblk = Mf + b * 16 * LDF + b * 16;
        float x[16], sv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[i] = (i == c) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          x[m] = sv[m];
#pragma unroll
          for (int i = m + 1; i < 16; ++i) sv[i] -= Mblk[i * LDF + m] * x[m];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) Tf[(b * 16 + i) * LDF + b * 16 + c] = x[i];
      }
      wave_lds_sync();
      // first doubling level, T21 = -T22 (M21 T11) for the pair: Y to the
      // wave's own scratch, then T21; right operands read k-major, tiles
      // formed transposed (a lane writes four consecutive columns of a row)
      const int rb = 32 * wave + 16, cb = 32 * wave;
      float* ys = Ysc + wave * 16 * LDYS;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      {
        Frag<16, float> fa, fb;
        fa.load(Mf + rb * LDF + cb, LDF);
        fb.load_kmajor(Tf + cb * LDF + cb, LDF);
        mma(acc, fb, fa);
      }
      *reinterpret_cast<float4*>(ys + acc_col() * LDYS + acc_row(0)) =
          float4{acc[0], acc[1], acc[2], acc[3]};
      wave_lds_sync();
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      {
        Frag<16, float> fa, fb;
        fa.load(Tf + rb * LDF + rb, LDF);
        fb.load_kmajor(ys, LDYS);
        mma(acc, fb, fa);
      }
      *reinterpret_cast<float4*>(Tf + (rb + acc_col()) * LDF + cb + acc_row(0)) =
          float4{-acc[0], -acc[1], -acc[2], -acc[3]};
    } else {
      // record: the gate prefix, the ratios P_C / P_{t+1} and P_C
      const int u = tid - 128;
      for (int e = u; e <= C; e += 128) out[G::R_LP + e] = lpv[e];
      if (u < C) out[G::R_CF + u] = expf(lpv[C] - lpv[u + 1]);
      if (u == 0) out[G::R_PC] = expf(lpv[C]);
    }
    __syncthreads();

    // ---- second doubling level: T21 = -T22 Y, Y = M21 T11 (32 x 32) ---------
    // One 16x16 tile of Y per wave; beside it, the record rows t < 32, which
    // the first level completed: g0 = T e and V = T diag(h) (V's blocks above
    // the block diagonal are zero and the chain never reads them, so they are
    // not written).
    constexpr int LDY = G::LDY;
    float* Ysh = Ysc;
    {
      const int rt = wave >> 1, c = wave & 1;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 32; kk += 16) {
        Frag<16, float> fa, fb;
        fa.load(Mf + (32 + rt * 16) * LDF + kk, LDF);
        fb.load_kmajor(Tf + kk * LDF + c * 16, LDF);
        mma(acc, fb, fa);
      }
      *reinterpret_cast<float4*>(Ysh + (rt * 16 + acc_col()) * LDY + c * 16 + acc_row(0)) =
          float4{acc[0], acc[1], acc[2], acc[3]};
    }
    {
      const int t = tid >> 3, q = tid & 7, c0 = 4 * q;
      float sg = 0.f;
      if ((c0 >> 4) <= (t >> 4)) {
        const float4 tr = *reinterpret_cast<const float4*>(Tf + t * LDF + c0);
        const float4 h4 = *reinterpret_cast<const float4*>(hv + c0);
        *reinterpret_cast<float4*>(out + G::R_V + t * C + c0) =
            float4{tr.x * h4.x, tr.y * h4.y, tr.z * h4.z, tr.w * h4.w};
        const float4 e4 = *reinterpret_cast<const float4*>(ev + c0);
        sg = tr.x * e4.x + tr.y * e4.y + tr.z * e4.z + tr.w * e4.w;
      }
      sg = group_sum<8>(sg);
      if (q == 0) out[G::R_G + t] = sg;
    }
    __syncthreads();
    {
      const int rt = wave >> 1, c = wave & 1;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 32; kk += 16) {
        Frag<16, float> fa, fb;
        fa.load(Tf + (32 + rt * 16) * LDF + 32 + kk, LDF);
        fb.load_kmajor(Ysh + kk * LDY + c * 16, LDY);
        mma(acc, fb, fa);
      }
      *reinterpret_cast<float4*>(Tf + (32 + rt * 16 + acc_col()) * LDF + c * 16 + acc_row(0)) =
          float4{-acc[0], -acc[1], -acc[2], -acc[3]};
    }
    __syncthreads();

    // ---- record rows t >= 32: g0 = T e, V = T diag(h) ------------------------
    {
      const int t = 32 + (tid >> 3), q = tid & 7;
      float sg = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c0 = 8 * q + 4 * h;
        if ((c0 >> 4) <= (t >> 4)) {
          const float4 tr = *reinterpret_cast<const float4*>(Tf + t * LDF + c0);
          const float4 h4 = *reinterpret_cast<const float4*>(hv + c0);
          *reinterpret_cast<float4*>(out + G::R_V + t * C + c0) =
              float4{tr.x * h4.x, tr.y * h4.y, tr.z * h4.z, tr.w * h4.w};
          const float4 e4 = *reinterpret_cast<const float4*>(ev + c0);
          sg += tr.x * e4.x + tr.y * e4.y + tr.z * e4.z + tr.w * e4.w;
        }
      }
      sg = group_sum<8>(sg);
      if (q == 0) out[G::R_G + t] = sg;
    }
    __syncthreads();  // the next chunk's split squares overwrite T
  }
}

// ---------------------------------------------------------------------------
// chain: the serial recurrence over the chunks of one (batch, head)
// ---------------------------------------------------------------------------
// Buffer resource over `bytes` bytes from `base` (raw, no stride); loads
// through it take a per-chunk scalar base and 32-bit per-lane offsets that
// stay the same from one chunk to the next.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Two consecutive key channels of one token as one LDS read (the d update
// reads the keys by channel pair).
template <typename Tin>
struct KeyPair;
template <>
struct KeyPair<__bf16> {
  using T = unsigned;
  __device__ static float lo(T p) { return __uint_as_float(p << 16); }
  __device__ static float hi(T p) { return __uint_as_float(p & 0xffff0000u); }
};
template <>
struct KeyPair<float> {
  using T = float2;
  __device__ static float lo(T p) { return p.x; }
  __device__ static float hi(T p) { return p.y; }
};

// Waves of the chain workgroup: 8 where every section still has whole
// 16-byte key loads and a supported lane reduction, else 4.
template <int DK>
constexpr int chain_waves() { return DK >= 64 ? 8 : 4; }

template <int DK, typename Tin>
struct ChainRegs {
  using G = P1Cfg<DK, Tin>;
  static constexpr int C = G::C, NW = chain_waves<DK>(), NT = 64 * NW;
  // x and g: TPR threads per token row t = tid / TPR; part q = tid % TPR
  // holds channels [q SEG1, (q+1) SEG1) of the key and block q (NV wide) of
  // the row of V.
  static constexpr int TPR = NT / C;
  static constexpr int SEG1 = DK / TPR;
  static constexpr int VEC = 16 / (int)sizeof(Tin);
  static constexpr int NR1 = SEG1 / VEC;
  static constexpr int NV = C / TPR;
  static_assert(NR1 >= 1 && SEG1 % VEC == 0 && NV % 4 == 0, "whole 16-byte loads");
  // d update: wave w owns channels [w DK/NW, (w+1) DK/NW) as NP pairs; lane l
  // takes pair l % NP over the RS3 token rows of segment l / NP.
  static constexpr int NP = DK / (2 * NW), NSG = 64 / NP, RS3 = C / NSG;
  static_assert(NP == 4 || NP == 8 || NP == 16, "strided lane reduction");
  using Pair = typename KeyPair<Tin>::T;
  static constexpr unsigned ES = sizeof(Tin);
  // The chunk's raw keys, copied to LDS by the x section (which loads each
  // row slice once) for the d update: DW dwords per row, unpadded, each row
  // rotated by ROT dwords per d-update segment of its token, so that the 64
  // lanes of a d-update read (NSG segments x NP pairs) meet 64 different
  // banks; rotations are multiples of 4 dwords, so 16-byte writes stay
  // aligned and whole.
  static constexpr int DW = DK * (int)sizeof(Tin) / 4;
  static constexpr int PDW = (int)sizeof(Tin) / 2;  // dwords per channel pair
  static constexpr int ROT = NP * PDW;
  static_assert(ROT % 4 == 0, "rotation keeps 16-byte pieces whole");
  __device__ __forceinline__ static int kpos(int t, int dw) {
    return t * DW + ((dw + ROT * (t / RS3)) & (DW - 1));
  }

  uint4 kr[NR1];
  float4 vr[NV / 4];
  float g0, cf, pc;

  // Chunk operands, through buffer resources based at the chunk's first key
  // row (rk) and at its record (rr). TAIL: the chunk holds `valid` < C rows;
  // rows past the end read the last valid row instead (their step size is
  // zero, so they add nothing), which keeps the loads unconditional.
  template <bool TAIL>
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rr,
                                       int valid, int t, int q) {
    const unsigned row = TAIL ? (unsigned)min(t, valid - 1) : (unsigned)t;
#pragma unroll
    for (int i = 0; i < NR1; ++i)
      kr[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     rk, (row * DK + (unsigned)(q * SEG1 + i * VEC)) * ES, 0, 0));
    // V is zero above its 16 x 16 block diagonal (and not written there):
    // lanes whose columns lie beyond row t's block read the start of the row
    // instead and hold zeros, so that every lane issues the same loads and
    // the compiler can count them
    const bool vlive = NV * q < 16 * (t / 16 + 1);
    const unsigned vcol = vlive ? (unsigned)(NV * q) : 0u;
#pragma unroll
    for (int i = 0; i < NV / 4; ++i) {
      const float4 x = __builtin_bit_cast(
          float4, __builtin_amdgcn_raw_buffer_load_b128(
                      rr, (unsigned)(G::R_V + t * C + vcol + 4 * i) * 4u, 0, 0));
      vr[i] = vlive ? x : float4{0.f, 0.f, 0.f, 0.f};
    }
    g0 = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rr, (unsigned)(G::R_G + t) * 4u, 0, 0));
    cf = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rr, (unsigned)(G::R_CF + t) * 4u, 0, 0));
    pc = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rr, (unsigned)G::R_PC * 4u, 0, 0));
  }
};

template <int DK, typename Tin>
__global__ __launch_bounds__(64 * chain_waves<DK>()) void precond_chain_kernel(
    int T, int nchunks, const Tin* __restrict__ k, const float* __restrict__ d0in,
    float* __restrict__ rec, float* __restrict__ dent, float* __restrict__ dT) {
  using G = P1Cfg<DK, Tin>;
  using R = ChainRegs<DK, Tin>;
  using KP = KeyPair<Tin>;
  constexpr int C = G::C, NT = R::NT, TPR = R::TPR;
  __shared__ __attribute__((aligned(16))) float dv[DK];
  __shared__ float xs[C], cgs[C];
  __shared__ __attribute__((aligned(16))) unsigned Ks[C * R::DW];
  const int bh = blockIdx.x, tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int t = tid / TPR, q = tid % TPR;
  const int sg = lane / R::NP;
  const int c3 = wave * (DK / R::NW) + 2 * (lane % R::NP);

  const Tin* kb = k + (size_t)bh * T * DK;
  float* recb = rec + (size_t)bh * nchunks * G::RS;
  float* dentb = dent + (size_t)bh * nchunks * DK;
  for (int c = tid; c < DK; c += NT) {
    const float x = d0in ? d0in[(size_t)bh * DK + c] : 1.f;
    dv[c] = x;
    if (nchunks > 0) dentb[c] = x;  // d at the entry of chunk 0
  }
  __syncthreads();

  const int nfull = T / C;  // chunks with C valid rows
  auto fetch_chunk = [&](R& r, int jj) {
    const int valid = min(C, T - jj * C);
    const auto rk = chunk_rsrc(kb + (size_t)jj * C * DK, (unsigned)(valid * DK) * R::ES);
    const auto rr = chunk_rsrc(recb + (size_t)jj * G::RS, (unsigned)G::RS * 4u);
    if (jj < nfull)
      r.template load<false>(rk, rr, C, t, q);
    else
      r.template load<true>(rk, rr, valid, t, q);
  };
  // One chunk: `cur` holds chunk jj (fetched two chunks before); chunk jj + 2
  // is fetched into `fetch` at the start (the last chunk again near the end).
  auto step = [&](int jj, R& fetch, const R& cur) {
    fetch_chunk(fetch, min(jj + 2, nchunks - 1));
    float* rc = recb + (size_t)jj * G::RS;
    // x_t = <d, a_t>; the key row slice also goes to LDS for the d update
    {
      const Tin* kv = reinterpret_cast<const Tin*>(cur.kr);
#pragma unroll
      for (int i = 0; i < R::NR1; ++i)
        *reinterpret_cast<uint4*>(Ks + R::kpos(t, (q * R::NR1 + i) * 4)) = cur.kr[i];
      const float* dq = dv + q * R::SEG1;
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int c = 0; c < R::SEG1; c += 2) {
        const float x0 = to_f32(kv[c]), x1 = to_f32(kv[c + 1]);
        s0 += x0 * x0 * dq[c];
        s1 += x1 * x1 * dq[c + 1];
      }
      const float s = group_sum<TPR>(s0 + s1);
      if (q == 0) xs[t] = s;
    }
    __syncthreads();
    // g_t = g0_t - sum_i V[t][i] x_i
    {
      const float* vv = reinterpret_cast<const float*>(cur.vr);
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < R::NV; ++i) s += vv[i] * xs[R::NV * q + i];
      s = group_sum<TPR>(s);
      const float g = cur.g0 - s;
      if (q == 0) {
        rc[G::R_G + t] = g;
        cgs[t] = cur.cf * g;
      }
    }
    __syncthreads();
    // d <- P_C d + sum_t a_t (c_t g_t); the new d is the next chunk's entry
    {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int m = 0; m < R::RS3; ++m) {
        const int tt = sg * R::RS3 + m;
        const float cg = cgs[tt];
        const typename R::Pair kp = *reinterpret_cast<const typename R::Pair*>(
            Ks + R::kpos(tt, c3 * R::PDW / 2));
        const float x0 = KP::lo(kp), x1 = KP::hi(kp);
        s0 += x0 * x0 * cg;
        s1 += x1 * x1 * cg;
      }
      s0 = strided_sum<R::NP>(s0);
      s1 = strided_sum<R::NP>(s1);
      if (sg == 0) {
        const float2 od = *reinterpret_cast<const float2*>(dv + c3);
        const float2 nd = float2{cur.pc * od.x + s0, cur.pc * od.y + s1};
        *reinterpret_cast<float2*>(dv + c3) = nd;
        if (jj + 1 < nchunks)
          *reinterpret_cast<float2*>(dentb + (size_t)(jj + 1) * DK + c3) = nd;
      }
    }
    __syncthreads();
  };
  // Three register sets in turn (chunk jj uses set jj % 3), unrolled so that
  // each set is a fixed object.
  R ra, rb, rc3;
  if (nchunks > 0) {
    fetch_chunk(ra, 0);
    fetch_chunk(rb, min(1, nchunks - 1));
  }
  int jj = 0;
  for (; jj + 2 < nchunks; jj += 3) {
    step(jj, rc3, ra);
    step(jj + 1, ra, rb);
    step(jj + 2, rb, rc3);
  }
  if (jj < nchunks) step(jj++, rc3, ra);
  if (jj < nchunks) step(jj++, ra, rb);
  if (dT && tid < DK) dT[(size_t)bh * DK + tid] = dv[tid];
}

// ---------------------------------------------------------------------------
// ktilde: K~ = (P d0^T + L A) * K per chunk
// ---------------------------------------------------------------------------
template <int DK, typename Tin>
__global__ __launch_bounds__(256) void precond_ktilde_kernel(
    int T, int nchunks, const Tin* __restrict__ k, const float* __restrict__ rec,
    const float* __restrict__ dent, Tin* __restrict__ ktil) {
  using G = P1Cfg<DK, Tin>;
  constexpr int C = G::C, LDK = G::LDK, LDC = G::LDC, VEC = G::VEC, NCB = G::NCB,
                DB = G::DB;
  __shared__ __attribute__((aligned(16))) unsigned char smem[G::kt_bytes];
  Tin* Ks = reinterpret_cast<Tin*>(smem + G::kK);
  Tin* As = reinterpret_cast<Tin*>(smem + G::kA);
  Tin* Lb = reinterpret_cast<Tin*>(smem + G::kL);
  float* lpv = reinterpret_cast<float*>(smem + G::kVec);  // C + 4
  float* Pv = lpv + C + 4;
  float* gv = Pv + C;
  float* dv = gv + C;

  const int bh = blockIdx.x / nchunks, j = blockIdx.x - bh * nchunks;
  const int tid = threadIdx.x, wave = wave_id();
  const int valid = min(C, T - j * C);
  const size_t t0 = (size_t)bh * T + (size_t)j * C;
  const float* rc = rec + (size_t)blockIdx.x * G::RS;

#pragma unroll
  for (int i = 0; i < G::NLK; ++i) {
    const int e = tid + i * G::NT;
    const int rr = e / NCB, cc = (e % NCB) * VEC;
    uint4 kr = {0u, 0u, 0u, 0u};
    if (rr < valid) kr = *reinterpret_cast<const uint4*>(k + (t0 + rr) * DK + cc);
    *reinterpret_cast<uint4*>(Ks + rr * LDK + cc) = kr;
    const Tin* kv = reinterpret_cast<const Tin*>(&kr);
    Tin a[VEC];
#pragma unroll
    for (int u = 0; u < VEC; ++u) {
      const float x = to_f32(kv[u]);
      a[u] = from_f32<Tin>(x * x);
    }
    *reinterpret_cast<uint4*>(As + rr * LDK + cc) = *reinterpret_cast<const uint4*>(a);
  }
  if (tid <= C) lpv[tid] = rc[G::R_LP + tid];
  if (tid < C) gv[tid] = rc[G::R_G + tid];
  if (tid < DK) dv[tid] = dent[(size_t)blockIdx.x * DK + tid];
  __syncthreads();
  if (tid < C) Pv[tid] = expf(lpv[tid]);
  // four consecutive entries of a row per thread and access
  for (int e4 = tid; e4 < C * C / 4; e4 += G::NT) {
    const int tt = e4 / (C / 4), i0 = (e4 % (C / 4)) * 4;
    Tin lv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u;
      lv[u] = from_f32<Tin>(i < tt ? __expf(lpv[tt] - lpv[i + 1]) * gv[i] : 0.f);
    }
    if constexpr (sizeof(Tin) == 2)
      *reinterpret_cast<uint2*>(Lb + tt * LDC + i0) = *reinterpret_cast<const uint2*>(lv);
    else
      *reinterpret_cast<uint4*>(Lb + tt * LDC + i0) = *reinterpret_cast<const uint4*>(lv);
  }
  __syncthreads();
  // wave w: token block w, all channel blocks; K~ overwrites K in place (each
  // element is read and written by the same lane)
  {
    const int tb = wave;
    Frag<C, Tin> fl;
    fl.load(Lb + tb * 16 * LDC, LDC);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      Frag<C, Tin> fa;
      fa.load_kmajor(As + db * 16, LDK);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mma(acc, fl, fa);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = tb * 16 + acc_row(i), c = db * 16 + acc_col();
        const float dt = Pv[tt] * dv[c] + acc[i];
        Ks[tt * LDK + c] = from_f32<Tin>(dt * to_f32(Ks[tt * LDK + c]));
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < G::NLK; ++i) {
    const int e = tid + i * G::NT;
    const int rr = e / NCB, cc = (e % NCB) * VEC;
    if (rr < valid)
      *reinterpret_cast<uint4*>(ktil + (t0 + rr) * DK + cc) =
          *reinterpret_cast<const uint4*>(Ks + rr * LDK + cc);
  }
}

// ---------------------------------------------------------------------------
// rho: the per-token residual contraction ratio and its geometric mean
// ---------------------------------------------------------------------------
// [OSDN-it] section 3 (Theorem 5.2): f_t(S_t) / f_t(S_{t-1}) =
// (1 - beta_t c_t)^2 with c_t = <d_t, a_t>; section 4.2 reports its geometric
// mean q_geo. From the chain's step sizes, 1 - beta_t c_t = g_t / e_t where
// e_t = eta beta_t / n_t is nonzero; otherwise (eta = 0, beta_t = 0 or a zero
// key) no step has been taken inside the chunk before t that the ratio could
// see, so c_t = P_t <d_entry, a_t> exactly. One workgroup per (batch, head),
// one token per thread, the entry values of d of the four chunks a block of
// 256 tokens spans staged in LDS. Runs after the chain; reads its records.
template <int DK, typename Tin>
__global__ __launch_bounds__(256) void precond_rho_kernel(
    int T, int nchunks, const Tin* __restrict__ k, const float* __restrict__ beta,
    float eta, const float* __restrict__ rec, const float* __restrict__ dent,
    float* __restrict__ rho, float* __restrict__ qgeo) {
  using G = P1Cfg<DK, Tin>;
  constexpr int C = G::C, VEC = G::VEC, NB = 256 / C;
  __shared__ float dsh[NB * DK];
  __shared__ float red[4];
  const int bh = blockIdx.x, tid = threadIdx.x;
  float lsum = 0.f;
  for (int t0 = 0; t0 < T; t0 += 256) {
    const int j0 = t0 / C;
    for (int e = tid; e < NB * DK; e += 256) {
      const int jc = j0 + e / DK;
      dsh[e] = jc < nchunks ? dent[((size_t)bh * nchunks + jc) * DK + e % DK] : 0.f;
    }
    __syncthreads();
    const int t = t0 + tid;
    if (t < T) {
      const int j = t / C, i = t % C;
      const float* dd = dsh + (j - j0) * DK;
      const Tin* kr = k + ((size_t)bh * T + t) * DK;
      float n = 0.f, x = 0.f;
#pragma unroll
      for (int c = 0; c < DK; c += VEC) {
        const uint4 u = *reinterpret_cast<const uint4*>(kr + c);
        const Tin* kv = reinterpret_cast<const Tin*>(&u);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float kx = to_f32(kv[e]);
          const float a = kx * kx;
          n += a;
          x += a * dd[c + e];
        }
      }
      const float bt = beta[(size_t)bh * T + t];
      const float et = n > 0.f ? eta * bt / n : 0.f;
      const float* rc = rec + ((size_t)bh * nchunks + j) * G::RS;
      const float y = et != 0.f ? rc[G::R_G + i] / et
                                : 1.f - bt * expf(rc[G::R_LP + i]) * x;
      const float rt = y * y;
      if (rho) rho[(size_t)bh * T + t] = rt;
      lsum += logf(rt);
    }
    __syncthreads();
  }
  lsum = wave_sum(lsum);
  if ((tid & 63) == 0) red[tid >> 6] = lsum;
  __syncthreads();
  if (tid == 0 && qgeo)
    qgeo[bh] = T > 0 ? expf((red[0] + red[1] + red[2] + red[3]) / (float)T) : 1.f;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static int nchunks_of(int T) { return (T + kPrecondChunk - 1) / kPrecondChunk; }

template <int DK, typename Tin>
static size_t ws_floats(int BH, int T) {
  return (size_t)BH * nchunks_of(T) * (P1Cfg<DK, Tin>::RS + DK);
}

template <int DK, typename Tin>
static int launch_dk(const PrecondArgs& a, hipStream_t s) {
  using G = P1Cfg<DK, Tin>;
  static_assert(G::TB == G::NW, "one token block per wave in the ktilde kernel");
  const int BH = a.B * a.H, nch = nchunks_of(a.T);
  float* rec = static_cast<float*>(a.ws);
  float* dent = rec + (size_t)BH * nch * G::RS;
  const dim3 block(256);
  if (nch > 0) {
    const int tk_prep = ktimer_before(s, "precond_prep");
    // persistent grid of two workgroups per compute unit: three fit by LDS,
    // but two measured faster (at 4096 and at 2048 chunks the prep took
    // 65 and 36 us with two per unit against 76 and 40 us with three, and
    // 69 and 39 us with one workgroup per chunk)
    constexpr int per_cu = 2;
    static_assert(per_cu * G::prep_bytes <= 163840, "LDS");
    const int total = BH * nch;
    const int grid = total < 256 * per_cu ? total : 256 * per_cu;
    hipLaunchKernelGGL((precond_prep_kernel<DK, Tin>), dim3(grid), block, 0, s,
                       a.T, nch, total, (const Tin*)a.k, a.beta, a.r, a.eta, rec);
    ktimer_after(s, tk_prep);
    const int rc = (int)hipGetLastError();
    if (rc) return rc;
  }
  const int tk_chain = ktimer_before(s, "precond_chain");
  hipLaunchKernelGGL((precond_chain_kernel<DK, Tin>), dim3(BH), dim3(64 * chain_waves<DK>()), 0, s, a.T,
                     nch, (const Tin*)a.k, a.d0, rec, dent, a.dT);
  ktimer_after(s, tk_chain);
  int rc = (int)hipGetLastError();
  if (rc) return rc;
  if (a.rho || a.qgeo) {
    const int tk_rho = ktimer_before(s, "precond_rho");
    hipLaunchKernelGGL((precond_rho_kernel<DK, Tin>), dim3(BH), block, 0, s, a.T, nch,
                       (const Tin*)a.k, a.beta, a.eta, rec, dent, a.rho, a.qgeo);
    ktimer_after(s, tk_rho);
    rc = (int)hipGetLastError();
    if (rc) return rc;
  }
  if (nch > 0 && a.ktilde) {
    const int tk_ktilde = ktimer_before(s, "precond_ktilde");
    hipLaunchKernelGGL((precond_ktilde_kernel<DK, Tin>), dim3(BH * nch), block, 0, s,
                       a.T, nch, (const Tin*)a.k, rec, dent, (Tin*)a.ktilde);
    ktimer_after(s, tk_ktilde);
    rc = (int)hipGetLastError();
  }
  return rc;
}

size_t precond_workspace_bytes(int B, int H, int T, int Dk, int bf16) {
  const int BH = B * H;
  size_t f = 0;
  if (bf16) {
    switch (Dk) {
      case 32: f = ws_floats<32, __bf16>(BH, T); break;
      case 64: f = ws_floats<64, __bf16>(BH, T); break;
      case 128: f = ws_floats<128, __bf16>(BH, T); break;
    }
  } else {
    switch (Dk) {
      case 32: f = ws_floats<32, float>(BH, T); break;
      case 64: f = ws_floats<64, float>(BH, T); break;
      case 128: f = ws_floats<128, float>(BH, T); break;
    }
  }
  return f * 4;
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
