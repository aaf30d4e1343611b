// Recurrent decode: a few tokens advanced through the token recurrence itself,
// with the state read once from HBM, kept in registers and written back in
// place. This is the constant-memory inference regime of linear attention
// ([OSDN-it] section 1 and 4.3; [GDN2-it] method part 1), where a step is
// bound by streaming the Dk x Dv fp32 state.
//
// One workgroup (4 waves) per (batch, head). A state row is spread over an
// aligned group of 16 lanes, each lane holding D/16 of its columns (16-byte
// pieces 64 columns apart, so each load instruction of a group covers 256
// contiguous bytes of the row); the 16 row groups of the workgroup take rows
// g, g + 16, ... Reductions along a row are row-of-16 DPP sums.
//
// OSDN (state [Dv, Dk], row = value channel):
//   a = k*k, n = ||k||^2, c = <d, a>, k~ = d*k         (lane-local, 16-lane sums)
//   S <- S Diag(alpha)                                 (decaying backbone only)
//   S <- S + beta (v - S k) k~^T, o = scale S q        (per row, 16-lane sums)
//   d <- r d + eta beta (1 - beta c)/n a              (0 step if n = 0)
// Every row group tracks d for its own columns, so d needs no exchange.
// GDN-2 (state [Dk, Dv], row = key channel): the sums run over rows, i.e.
// over the lane groups of a wave (cross-row swaps) and then over the four
// waves through LDS, two barriers per token.
#include "device_common.hpp"
#include "launch.hpp"
#include "row_state.hpp"

namespace osdn {
namespace {

template <int DK, int DV, typename Tin>
__global__ __launch_bounds__(kDecThreads) void osdn_decode_kernel(
    int T, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const float* __restrict__ beta,
    const float* __restrict__ r, float eta, const float* __restrict__ log_alpha,
    float* __restrict__ S, float* __restrict__ d, float scale, Tin* __restrict__ o) {
  constexpr int NC = DK / 16, NR = DV / 16;
  const int bh = blockIdx.x;
  const int cl = threadIdx.x & 15, rg = threadIdx.x >> 4;
  float* Sb = S + (size_t)bh * DV * DK;
  float* db = d + (size_t)bh * DK;

  float s[NR][NC], dv[NC];
#pragma unroll
  for (int i = 0; i < NR; ++i) load_cols<DK, float>(Sb + (size_t)(rg + 16 * i) * DK, cl, s[i]);
  load_cols<DK, float>(db, cl, dv);

  const size_t tb = (size_t)bh * T;
  for (int t = 0; t < T; ++t) {
    const size_t tt = tb + t;
    float kk[NC], qq[NC], vv[NR];
    load_cols<DK, Tin>(k + tt * DK, cl, kk);
    load_cols<DK, Tin>(q + tt * DK, cl, qq);
#pragma unroll
    for (int i = 0; i < NR; ++i) vv[i] = to_f32(v[tt * DV + rg + 16 * i]);
    const float bt = beta[tt];
    const float rt = r ? r[tt] : 1.f;
    if (log_alpha) {
      // per-key-channel decay of the state before the token's step
      float la[NC];
      load_cols<DK, float>(log_alpha + tt * DK, cl, la);
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const float al = expf(la[j]);
#pragma unroll
        for (int i = 0; i < NR; ++i) s[i][j] *= al;
      }
    }

    // key statistics and the read S k, all with the plain key
    float n = 0.f, c = 0.f, kt[NC], p[NR];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const float a = kk[j] * kk[j];
      n += a;
      c += dv[j] * a;
      kt[j] = dv[j] * kk[j];
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < NC; ++j) acc += s[i][j] * kk[j];
      p[i] = acc;
    }
    n = row16_sum(n);
    c = row16_sum(c);
#pragma unroll
    for (int i = 0; i < NR; ++i) p[i] = row16_sum(p[i]);

    // write with the preconditioned key, then read out with q
    float ov[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float u = bt * (vv[i] - p[i]);
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        s[i][j] += u * kt[j];
        acc += s[i][j] * qq[j];
      }
      ov[i] = acc;
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) ov[i] = row16_sum(ov[i]);
#pragma unroll
    for (int i = 0; i < NR; ++i)
      if (cl == (i & 15)) o[tt * DV + rg + 16 * i] = from_f32<Tin>(scale * ov[i]);

    // preconditioner step (descent on the closed-form surrogate, gate r)
    const float g = n > 0.f ? eta * bt * (1.f - bt * c) / n : 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) dv[j] = rt * dv[j] + g * (kk[j] * kk[j]);
  }

#pragma unroll
  for (int i = 0; i < NR; ++i) store_cols<DK>(Sb + (size_t)(rg + 16 * i) * DK, cl, s[i]);
  // every thread has consumed its copy of d (T >= 1: the first token's sums
  // read it) before row group 0 overwrites it
  __syncthreads();
  if (rg == 0) store_cols<DK>(db, cl, dv);
}

template <int DK, int DV, typename Tin>
__global__ __launch_bounds__(kDecThreads) void gdn2_decode_kernel(
    int T, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const float* __restrict__ log_alpha,
    const Tin* __restrict__ bg, const Tin* __restrict__ wg,
    float* __restrict__ S, float scale, Tin* __restrict__ o) {
  constexpr int NR = DK / 16, NC = DV / 16;
  __shared__ float red[2][kDecThreads / kWave][DV];
  const int bh = blockIdx.x;
  const int cl = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  float* Sb = S + (size_t)bh * DK * DV;

  float s[NR][NC];
#pragma unroll
  for (int m = 0; m < NR; ++m) load_cols<DV, float>(Sb + (size_t)(rg + 16 * m) * DV, cl, s[m]);

  // sum over the 64 row groups' partials: the four groups of a wave by
  // cross-row swaps, then the four waves through LDS buffer `b`
  auto row_sum = [&](float (&x)[NC], int b) {
#pragma unroll
    for (int j = 0; j < NC; ++j) x[j] = add_swap32(add_swap16(x[j]));
    if (lane < 16) {
#pragma unroll
      for (int j = 0; j < NC; ++j) red[b][wave][dec_col<DV>(cl, j)] = x[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int col = dec_col<DV>(cl, j);
      x[j] = red[b][0][col] + red[b][1][col] + red[b][2][col] + red[b][3][col];
    }
  };

  const size_t tb = (size_t)bh * T;
  for (int t = 0; t < T; ++t) {
    const size_t tt = tb + t;
    float kk[NR], ee[NR], qq[NR], z[NC], vv[NC];
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const size_t e = tt * DK + rg + 16 * m;
      kk[m] = to_f32(k[e]);
      ee[m] = to_f32(bg[e]) * kk[m];
      qq[m] = to_f32(q[e]);
      const float al = expf(log_alpha[e]);
#pragma unroll
      for (int j = 0; j < NC; ++j) s[m][j] *= al;
    }
    load_cols<DV, Tin>(v + tt * DV, cl, vv);
    load_cols<DV, Tin>(wg + tt * DV, cl, z);
#pragma unroll
    for (int j = 0; j < NC; ++j) z[j] *= vv[j];

    // erase the read S^T (b*k), write k (w*v)^T
    float rd[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < NR; ++m) acc += s[m][j] * ee[m];
      rd[j] = acc;
    }
    row_sum(rd, 0);
    float po[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const float u = z[j] - rd[j];
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < NR; ++m) {
        s[m][j] += kk[m] * u;
        acc += s[m][j] * qq[m];
      }
      po[j] = acc;
    }
    row_sum(po, 1);
    if (threadIdx.x < 16) {
#pragma unroll
      for (int j = 0; j < NC; ++j)
        o[tt * DV + dec_col<DV>(cl, j)] = from_f32<Tin>(scale * po[j]);
    }
  }

#pragma unroll
  for (int m = 0; m < NR; ++m) store_cols<DV>(Sb + (size_t)(rg + 16 * m) * DV, cl, s[m]);
}

template <int DK, int DV, typename Tin>
int launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  const int tk = ktimer_before(s, a.gdn2 ? "gdn2_decode" : "osdn_decode");
  if (a.gdn2) {
    hipLaunchKernelGGL((gdn2_decode_kernel<DK, DV, Tin>), dim3(BH), dim3(kDecThreads), 0, s,
                       a.T, (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.v, a.log_alpha,
                       (const Tin*)a.b, (const Tin*)a.w, a.S, a.scale, (Tin*)a.o);
  } else {
    hipLaunchKernelGGL((osdn_decode_kernel<DK, DV, Tin>), dim3(BH), dim3(kDecThreads), 0, s,
                       a.T, (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.v, a.beta, a.r,
                       a.eta, a.log_alpha, a.S, a.d, a.scale, (Tin*)a.o);
  }
  ktimer_after(s, tk);
  return (int)hipGetLastError();
}

template <int DK, typename Tin>
int launch_decode_dv(const DecodeArgs& a, hipStream_t s) {
  switch (a.Dv) {
    case 32: return launch_decode_t<DK, 32, Tin>(a, s);
    case 64: return launch_decode_t<DK, 64, Tin>(a, s);
    case 128: return launch_decode_t<DK, 128, Tin>(a, s);
  }
  return -1;
}

template <typename Tin>
int launch_decode_dk(const DecodeArgs& a, hipStream_t s) {
  switch (a.Dk) {
    case 32: return launch_decode_dv<32, Tin>(a, s);
    case 64: return launch_decode_dv<64, Tin>(a, s);
    case 128: return launch_decode_dv<128, Tin>(a, s);
  }
  return -1;
}

}  // namespace

int launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.B * a.H == 0 || a.T == 0) return 0;
  return a.bf16 ? launch_decode_dk<__bf16>(a, s) : launch_decode_dk<float>(a, s);
}

}  // namespace osdn
