// Pieces shared by the backward kernels of backward.hip (OSDN) and
// backward_gated.hip (GDN-2, OSDN on a decaying backbone): the split of a
// stream's value rows into workgroup slices, the layout of the per-token
// row sums the slices hand over, and the kernel that adds those sums and
// carries the adjoint of OSDN's preconditioner learner ([OSDN-it] sections
// 2.2-2.3) backwards over the tokens.
#pragma once

#include "device_common.hpp"
#include "row_state.hpp"

namespace osdn {

constexpr int kCkpt = 64;                         // tokens between stored states
constexpr int kBwdNR = 2;                         // value rows per thread
constexpr int kBwdThreads = 256;                  // 16 row groups x 16 column lanes
constexpr int kBwdRG = kBwdThreads / 16;          // row groups
constexpr int kBwdSliceRows = kBwdRG * kBwdNR;    // value rows per workgroup

__host__ __device__ inline int nckpt(int T) { return (T + kCkpt - 1) / kCkpt; }
// Per token and slice, the slice's sums over its rows: S^T do, dS^T u,
// S_{t-1}^T w (Dk each), u.w and (gated) u.do, padded to 3 Dk + 4; the gated
// rule adds the decay's column sums of dS_dec * S_dec (Dk).
__host__ __device__ constexpr int share_width(int Dk, bool gated) {
  return 3 * Dk + 4 + (gated ? Dk : 0);
}

// Workgroup -> (stream, slice): the slices of a stream are 8 workgroups
// apart, so that workgroups dispatched round-robin over the eight XCDs put
// all of a stream's slices on one XCD (they read the same keys and queries).
__device__ __forceinline__ void slice_of(int RS, int& bh, int& sl) {
  const int x = blockIdx.x, grp = x / (8 * RS), rr = x % (8 * RS);
  sl = rr / 8;
  bh = grp * 8 + rr % 8;
}
inline int bwd_grid(int BH, int RS) { return ((BH + 7) / 8) * 8 * RS; }

// The learner's adjoint, one workgroup of four waves per stream. Wave 0
// walks the tokens backwards (lane l holds channels l + 64 m, m < LM; at
// Dk = 32 the upper half of the wave holds zeros) while waves 1-3 stage the
// next block of kLearnBlock tokens in LDS: the slices' shares added up, d_t,
// the key, beta and r. One barrier per block.
constexpr int kLearnBlock = 16;
constexpr int kLearnThreads = 256;

struct LearnerArgs {
  int T;
  const void* k;
  const float *beta, *r;
  float eta, scale;
  const float* ddT;
  const float* d;    // d_t per token [B*H][T][Dk]
  const float* sh;   // shares [B*H][T][RS][SW]
  float *gq, *gk, *gbeta, *gr, *geta, *gd0;
  float* gla;        // GATED: the decay's gradient [B*H][T][Dk]
};

template <int DK, int DV, typename Tin, bool GATED>
__global__ __launch_bounds__(kLearnThreads) void osdn_bwd_learner_kernel(LearnerArgs p) {
  constexpr int LM = DK >= 64 ? DK / 64 : 1, RS = DV / kBwdSliceRows;
  constexpr int SW = share_width(DK, GATED);
  const int T = p.T;
  const Tin* k = (const Tin*)p.k;
  const float* beta = p.beta;
  const float* r = p.r;
  const float eta = p.eta, scale = p.scale;
  constexpr int LB = kLearnBlock;
  // staged token: shares [0, SH) (S^T do, dS^T u, S_{t-1}^T w, u.w, and for
  // the gated rule u.do), d_t [SH, SH + DK), key [SH + DK, SH + 2 DK), beta
  // and r after them; the gated rule's decay sums go straight to their
  // output
  constexpr int SH = 3 * DK + 4;
  constexpr int OD = SH, OK = SH + DK, OB = SH + 2 * DK, TW = SH + 2 * DK + 4;
  static_assert(kLearnThreads - kWave >= LB, "a staging thread per token for beta and r");
  // staging: 16-byte pieces per token of the shares (NSH, each the sum of
  // RS slices), of d_t and of the key (ND each); one item type per loop, so
  // that every lane of a loop issues the same loads
  constexpr int NSH = SH / 4, ND = DK / 4;
  constexpr int NL = kLearnThreads - kWave;            // staging threads
  constexpr int NIS = (LB * NSH + NL - 1) / NL;        // share items per thread
  constexpr int NIK = (LB * ND + NL - 1) / NL;         // d_t or key items per thread
  __shared__ __attribute__((aligned(16))) float stg[2][LB][TW];
  const int bh = blockIdx.x, tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const float* Db = p.d + (size_t)bh * T * DK;
  const float* Sh = p.sh + (size_t)bh * T * RS * SW;
  const size_t tb = (size_t)bh * T;
  const int nblk = (T + LB - 1) / LB;

  // block b holds tokens T - 1 - b LB - i, i < LB (those below 0 are not
  // staged); every load is unconditional, of a clamped item and token, and
  // all are issued before the first LDS write
  auto stage = [&](int b, int buf) {
    const int st = tid - kWave;
    auto tok = [&](int i) { return max(T - 1 - b * LB - i, 0); };
    float4 vs[NIS][RS], vd[NIK], vk[NIK];
    float2 vb = float2{0.f, 1.f};
#pragma unroll
    for (int u = 0; u < NIS; ++u) {
      const int it = min(st + u * NL, LB * NSH - 1), i = it / NSH, e = it - i * NSH;
      const float* sh = Sh + (size_t)tok(i) * RS * SW + 4 * e;
#pragma unroll
      for (int sl = 0; sl < RS; ++sl) vs[u][sl] = *reinterpret_cast<const float4*>(sh + sl * SW);
    }
#pragma unroll
    for (int u = 0; u < NIK; ++u) {
      const int it = min(st + u * NL, LB * ND - 1), i = it / ND, e = it - i * ND;
      const size_t t = (size_t)tok(i);
      vd[u] = *reinterpret_cast<const float4*>(Db + t * DK + 4 * e);
      const Tin* kp = k + (tb + t) * DK + 4 * e;
      vk[u] = float4{to_f32(kp[0]), to_f32(kp[1]), to_f32(kp[2]), to_f32(kp[3])};
    }
    {
      const size_t t = (size_t)tok(min(st, LB - 1));
      vb = float2{beta[tb + t], r ? r[tb + t] : 1.f};
    }
#pragma unroll
    for (int u = 0; u < NIS; ++u) {
      const int it = st + u * NL, i = it / NSH, e = it - i * NSH;
      float4 a = vs[u][0];
#pragma unroll
      for (int sl = 1; sl < RS; ++sl) {
        a.x += vs[u][sl].x;
        a.y += vs[u][sl].y;
        a.z += vs[u][sl].z;
        a.w += vs[u][sl].w;
      }
      if (it < LB * NSH) *reinterpret_cast<float4*>(&stg[buf][i][4 * e]) = a;
    }
#pragma unroll
    for (int u = 0; u < NIK; ++u) {
      const int it = st + u * NL, i = it / ND, e = it - i * ND;
      if (it < LB * ND) {
        *reinterpret_cast<float4*>(&stg[buf][i][OD + 4 * e]) = vd[u];
        *reinterpret_cast<float4*>(&stg[buf][i][OK + 4 * e]) = vk[u];
      }
    }
    if (st < LB) *reinterpret_cast<float2*>(&stg[buf][st][OB]) = vb;
    if constexpr (GATED) {
      // the decay's gradient: the slices' sums of dS_dec * S_dec
#pragma unroll
      for (int u = 0; u < NIK; ++u) {
        const int it = st + u * NL, i = min(it, LB * ND - 1) / ND;
        const int e = min(it, LB * ND - 1) - i * ND, t = T - 1 - b * LB - i;
        const float* sh = Sh + (size_t)max(t, 0) * RS * SW + SH + 4 * e;
        float4 a = *reinterpret_cast<const float4*>(sh);
#pragma unroll
        for (int sl = 1; sl < RS; ++sl) {
          const float4 x = *reinterpret_cast<const float4*>(sh + sl * SW);
          a.x += x.x;
          a.y += x.y;
          a.z += x.z;
          a.w += x.w;
        }
        if (it < LB * ND && t >= 0)
          *reinterpret_cast<float4*>(p.gla + (tb + t) * DK + 4 * e) = a;
      }
    }
  };

  float dd[LM];
#pragma unroll
  for (int m = 0; m < LM; ++m) {
    const int j = lane + 64 * m;
    dd[m] = (p.ddT && j < DK) ? p.ddT[(size_t)bh * DK + j] : 0.f;
  }
  float eta_acc = 0.f;

  auto compute = [&](int b, int buf) {
#pragma unroll 4
    for (int i = 0; i < LB; ++i) {
      const int t = T - 1 - b * LB - i;
      if (t < 0) break;
      const size_t tt = tb + t;
      const float* src = &stg[buf][i][0];
      float kk[LM], dt[LM], sq[LM], su[LM], sy[LM];
#pragma unroll
      for (int m = 0; m < LM; ++m) {
        // lanes past Dk read a valid channel and keep zeros
        const int j0 = lane + 64 * m, j = j0 < DK ? j0 : j0 - DK;
        const float live = j0 < DK ? 1.f : 0.f;
        kk[m] = live * src[OK + j];
        dt[m] = live * src[OD + j];
        su[m] = live * src[DK + j];
        sy[m] = live * src[2 * DK + j];
        sq[m] = live * src[j];
      }
      const float uw = src[3 * DK], bt = src[OB], rt = src[OB + 1];
      if constexpr (GATED) {
        // S_t^T do = S_dec^T do + beta k~ (u.do)
        const float ud = src[3 * DK + 1];
#pragma unroll
        for (int m = 0; m < LM; ++m) sq[m] += bt * dt[m] * kk[m] * ud;
      }

      float n = 0.f, c = 0.f, pr = 0.f, pg = 0.f;
      float a[LM], dk[LM], ddt[LM];
#pragma unroll
      for (int m = 0; m < LM; ++m) {
        a[m] = kk[m] * kk[m];
        n += a[m];
        c += dt[m] * a[m];
        // the write and the read of the memory: k~'s adjoint beta dS^T u,
        // the read key's -beta S_{t-1}^T w
        const float dkt = bt * su[m];
        dk[m] = -bt * sy[m] + dkt * dt[m];
        ddt[m] = dkt * kk[m] + rt * dd[m];
        pr += dd[m] * dt[m];
        pg += dd[m] * a[m];
      }
      n = wave_sum(n);
      c = wave_sum(c);
      const float drt = wave_sum(pr);
      const float dg = wave_sum(pg);
      // the learner's step g = eta beta (1 - beta c)/n, only where n > 0
      // (no step, no gradient through it, at a zero key)
      const float in = n > 0.f ? 1.f / n : 0.f;
      const float h = (1.f - bt * c) * in;   // (1 - beta c)/n
      const float g = eta * bt * h;
      const float hg = h * dg;
      const float dc = -eta * bt * bt * in * dg;
      const float dn = -g * in * dg;
      const float dbt = uw + eta * (1.f - 2.f * bt * c) * in * dg;
      eta_acc += bt * hg;
      float da[LM];
#pragma unroll
      for (int m = 0; m < LM; ++m) {
        ddt[m] += dc * a[m];
        da[m] = g * dd[m] + dc * dt[m] + dn;
      }
#pragma unroll
      for (int m = 0; m < LM; ++m) {
        const int j = lane + 64 * m;
        dk[m] += 2.f * kk[m] * da[m];
        dd[m] = ddt[m];
        if (DK >= 64 || j < DK) {
          p.gq[tt * DK + j] = scale * sq[m];
          p.gk[tt * DK + j] = dk[m];
        }
      }
      // (every lane holds the same sums; all store them, no branch)
      p.gbeta[tt] = dbt;
      p.gr[tt] = drt;
    }
  };

  if (nblk > 0 && wave > 0) stage(0, 0);
  __syncthreads();
  for (int b = 0; b < nblk; ++b) {
    if (wave > 0) {
      if (b + 1 < nblk) stage(b + 1, (b + 1) & 1);
    } else {
      compute(b, b & 1);
    }
    __syncthreads();
  }
  if (wave == 0) {
#pragma unroll
    for (int m = 0; m < LM; ++m) {
      const int j = lane + 64 * m;
      if (j < DK) p.gd0[(size_t)bh * DK + j] = dd[m];
    }
    if (lane == 0) p.geta[bh] = eta_acc;
  }
}

}  // namespace osdn
