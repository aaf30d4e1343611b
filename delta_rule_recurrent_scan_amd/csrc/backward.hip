// Backward pass of the OSDN forward: the reverse-mode adjoint of the token
// recurrence ([OSDN-it] sections 2.1-2.3), per (batch, head) and token t,
//   a = k_t*k_t, n = ||k_t||^2, c = <d_t, a>, k~ = d_t*k_t,
//   u = v_t - S_{t-1} k_t,  S_t = S_{t-1} + beta_t u k~^T,  o_t = scale S_t q_t,
//   g = eta beta_t (1 - beta_t c)/n (0 when n = 0),  d_{t+1} = r_t d_t + g a.
// Given the adjoints of o, S_T and d_T it produces those of q, k, v, beta, r,
// eta, d0 and S0: the memory update's adjoint and, through k~ and the
// learner's step, the adjoint of the phase-1 preconditioner scan.
//
// Two kernels, one workgroup (256 threads) per (batch, head), the state held
// in registers in the row layout of row_state.hpp:
//   record   runs the recurrence forward and stores, per token, the residual
//            u_t (Dv fp32) and the preconditioner d_t (Dk fp32), plus the
//            state every kCkpt tokens and after the last one (fp32);
//   reverse  walks the tokens backwards with S and its adjoint dS in
//            registers: S_{t-1} = S_t - beta_t u_t k~_t^T (reset exactly from
//            the stored state every kCkpt tokens), dS carried down.
// Per token, the sums over value rows (S_t^T do, dS^T u, S_{t-1}^T w, u.w)
// are the four row groups of a wave by cross-row swaps, then the four waves
// through LDS (one barrier, buffers alternating by token).
#include "device_common.hpp"
#include "launch.hpp"
#include "row_state.hpp"

namespace osdn {

constexpr int kCkpt = 64;  // tokens between stored states

__host__ __device__ inline int nckpt(int T) { return (T + kCkpt - 1) / kCkpt; }

size_t backward_workspace_bytes(int B, int H, int T, int Dk, int Dv) {
  const size_t BH = (size_t)B * H;
  return BH * ((size_t)T * (Dv + Dk) + (size_t)(nckpt(T) + 1) * Dv * Dk) * 4;
}

namespace {

struct BwdBufs {
  float *u, *d, *ck;
};

BwdBufs bwd_bufs(void* ws, int BH, int T, int Dk, int Dv) {
  float* f = static_cast<float*>(ws);
  BwdBufs b;
  b.u = f;
  b.d = b.u + (size_t)BH * T * Dv;
  b.ck = b.d + (size_t)BH * T * Dk;
  return b;
}

template <int DK, int DV, typename Tin>
__global__ __launch_bounds__(kDecThreads) void osdn_bwd_record_kernel(
    int T, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ beta, const float* __restrict__ r, float eta,
    const float* __restrict__ d0, const float* __restrict__ S0, BwdBufs wb) {
  constexpr int NC = DK / 16, NR = DV / 16;
  const int bh = blockIdx.x;
  const int cl = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int nck = nckpt(T);
  float* Ub = wb.u + (size_t)bh * T * DV;
  float* Db = wb.d + (size_t)bh * T * DK;
  float* Cb = wb.ck + (size_t)bh * (nck + 1) * DV * DK;

  float s[NR][NC], dv[NC];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    if (S0) {
      load_cols<DK, float>(S0 + ((size_t)bh * DV + rg + 16 * i) * DK, cl, s[i]);
    } else {
#pragma unroll
      for (int j = 0; j < NC; ++j) s[i][j] = 0.f;
    }
  }
  if (d0) {
    load_cols<DK, float>(d0 + (size_t)bh * DK, cl, dv);
  } else {
#pragma unroll
    for (int j = 0; j < NC; ++j) dv[j] = 1.f;
  }

  // the next token's inputs are loaded one token ahead, off the chain
  const size_t tb = (size_t)bh * T;
  float kn[NC], vn[NR], bn = 0.f, rn = 1.f;
  if (T > 0) {
    load_cols<DK, Tin>(k + tb * DK, cl, kn);
#pragma unroll
    for (int i = 0; i < NR; ++i) vn[i] = to_f32(v[tb * DV + rg + 16 * i]);
    bn = beta[tb];
    rn = r ? r[tb] : 1.f;
  }
  for (int t = 0; t < T; ++t) {
    if (t % kCkpt == 0) {
      float* C = Cb + (size_t)(t / kCkpt) * DV * DK;
#pragma unroll
      for (int i = 0; i < NR; ++i) store_cols<DK>(C + (size_t)(rg + 16 * i) * DK, cl, s[i]);
    }
    float kk[NC], vv[NR];
#pragma unroll
    for (int j = 0; j < NC; ++j) kk[j] = kn[j];
#pragma unroll
    for (int i = 0; i < NR; ++i) vv[i] = vn[i];
    const float bt = bn, rt = rn;
    if (t + 1 < T) {
      const size_t tn = tb + t + 1;
      load_cols<DK, Tin>(k + tn * DK, cl, kn);
#pragma unroll
      for (int i = 0; i < NR; ++i) vn[i] = to_f32(v[tn * DV + rg + 16 * i]);
      bn = beta[tn];
      rn = r ? r[tn] : 1.f;
    }
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
    if (rg == 0) store_cols<DK>(Db + (size_t)t * DK, cl, dv);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float u = vv[i] - p[i];
      if (cl == (i & 15)) Ub[(size_t)t * DV + rg + 16 * i] = u;
      const float bu = bt * u;
#pragma unroll
      for (int j = 0; j < NC; ++j) s[i][j] += bu * kt[j];
    }
    const float g = n > 0.f ? eta * bt * (1.f - bt * c) / n : 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) dv[j] = rt * dv[j] + g * (kk[j] * kk[j]);
  }
  float* C = Cb + (size_t)nck * DV * DK;
#pragma unroll
  for (int i = 0; i < NR; ++i) store_cols<DK>(C + (size_t)(rg + 16 * i) * DK, cl, s[i]);
}

template <int DK, int DV, typename Tin>
__global__ __launch_bounds__(kDecThreads) void osdn_bwd_kernel(
    int T, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const float* __restrict__ beta, const float* __restrict__ r, float eta, float scale,
    const Tin* __restrict__ dout, const float* __restrict__ dST,
    const float* __restrict__ ddT, BwdBufs wb, float* __restrict__ gq,
    float* __restrict__ gk, float* __restrict__ gv, float* __restrict__ gbeta,
    float* __restrict__ gr, float* __restrict__ geta, float* __restrict__ gd0,
    float* __restrict__ gS0) {
  constexpr int NC = DK / 16, NR = DV / 16, NW = kDecThreads / kWave;
  constexpr int RW = 3 * DK + 4;  // per wave: S^T do, dS^T u, S_{t-1}^T w, u.w
  __shared__ float red[2][NW][RW];
  const int bh = blockIdx.x;
  const int cl = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int nck = nckpt(T);
  const float* Ub = wb.u + (size_t)bh * T * DV;
  const float* Db = wb.d + (size_t)bh * T * DK;
  const float* Cb = wb.ck + (size_t)bh * (nck + 1) * DV * DK;

  // S after the last token, dS and the adjoint of d after it
  float s[NR][NC], ds[NR][NC], dd[NC];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    load_cols<DK, float>(Cb + (size_t)nck * DV * DK + (size_t)(rg + 16 * i) * DK, cl, s[i]);
    if (dST) {
      load_cols<DK, float>(dST + ((size_t)bh * DV + rg + 16 * i) * DK, cl, ds[i]);
    } else {
#pragma unroll
      for (int j = 0; j < NC; ++j) ds[i][j] = 0.f;
    }
  }
  if (ddT) {
    load_cols<DK, float>(ddT + (size_t)bh * DK, cl, dd);
  } else {
#pragma unroll
    for (int j = 0; j < NC; ++j) dd[j] = 0.f;
  }
  float eta_acc = 0.f;

  // the previous token's inputs are loaded one token ahead, off the chain
  const size_t tb = (size_t)bh * T;
  float kn[NC], qn[NC], dn_[NC], don[NR], un[NR], bn = 0.f, rn = 1.f;
  auto prefetch = [&](int t) {
    const size_t tt = tb + t;
    load_cols<DK, Tin>(k + tt * DK, cl, kn);
    load_cols<DK, Tin>(q + tt * DK, cl, qn);
    load_cols<DK, float>(Db + (size_t)t * DK, cl, dn_);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      don[i] = to_f32(dout[tt * DV + rg + 16 * i]);
      un[i] = Ub[(size_t)t * DV + rg + 16 * i];
    }
    bn = beta[tt];
    rn = r ? r[tt] : 1.f;
  };
  if (T > 0) prefetch(T - 1);
  for (int t = T - 1; t >= 0; --t) {
    const size_t tt = tb + t;
    float kk[NC], qq[NC], dt[NC], dov[NR], uu[NR];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      kk[j] = kn[j];
      qq[j] = qn[j];
      dt[j] = dn_[j];
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      dov[i] = don[i];
      uu[i] = un[i];
    }
    const float bt = bn, rt = rn;
    if (t > 0) prefetch(t - 1);
    float n = 0.f, c = 0.f, a[NC], kt[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      a[j] = kk[j] * kk[j];
      n += a[j];
      c += dt[j] * a[j];
      kt[j] = dt[j] * kk[j];
    }
    n = row16_sum(n);
    c = row16_sum(c);
    const float g = n > 0.f ? eta * bt * (1.f - bt * c) / n : 0.f;

    // o_t = scale S_t q_t:  dS += scale do q^T; then w = dS k~ (row sums)
    // and dS^T u (column partials)
    float w[NR], pu[NC], pq[NC], py[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) pu[j] = pq[j] = py[j] = 0.f;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float sd = scale * dov[i];
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        ds[i][j] += sd * qq[j];
        acc += ds[i][j] * kt[j];
        pu[j] += ds[i][j] * uu[i];
      }
      w[i] = acc;
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) w[i] = row16_sum(w[i]);
    // S_t^T do (column partials), then S_{t-1} = S_t - beta u k~^T (the
    // stored state at a checkpoint), S_{t-1}^T w, and dS_{t-1} = dS -
    // beta w k^T
    const bool ck = t % kCkpt == 0;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float bu = bt * uu[i], bw = bt * w[i];
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        pq[j] += s[i][j] * dov[i];
        s[i][j] -= bu * kt[j];
        ds[i][j] -= bw * kk[j];
      }
    }
    if (ck) {
      const float* C = Cb + (size_t)(t / kCkpt) * DV * DK;
#pragma unroll
      for (int i = 0; i < NR; ++i) load_cols<DK, float>(C + (size_t)(rg + 16 * i) * DK, cl, s[i]);
    }
    float pb = 0.f;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
#pragma unroll
      for (int j = 0; j < NC; ++j) py[j] += s[i][j] * w[i];
      pb += uu[i] * w[i];
    }
    pb = cl == 0 ? pb : 0.f;

    // sums over the 16 row groups: four per wave by swaps, four waves via LDS
    const int b = t & 1;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      pq[j] = add_swap32(add_swap16(pq[j]));
      pu[j] = add_swap32(add_swap16(pu[j]));
      py[j] = add_swap32(add_swap16(py[j]));
    }
    pb = wave_sum(pb);
    if (lane < 16) {
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const int col = dec_col<DK>(cl, j);
        red[b][wave][col] = pq[j];
        red[b][wave][DK + col] = pu[j];
        red[b][wave][2 * DK + col] = py[j];
      }
      if (lane == 0) red[b][wave][3 * DK] = pb;
    }
    __syncthreads();
    float sq[NC], su[NC], sy[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int col = dec_col<DK>(cl, j);
      sq[j] = su[j] = sy[j] = 0.f;
#pragma unroll
      for (int m = 0; m < NW; ++m) {
        sq[j] += red[b][m][col];
        su[j] += red[b][m][DK + col];
        sy[j] += red[b][m][2 * DK + col];
      }
    }
    float uw = 0.f;
#pragma unroll
    for (int m = 0; m < NW; ++m) uw += red[b][m][3 * DK];

    // adjoints of v, q; of k~ and k through the write and the read
#pragma unroll
    for (int i = 0; i < NR; ++i)
      if (cl == (i & 15)) gv[tt * DV + rg + 16 * i] = bt * w[i];
    float dk[NC], ddt[NC], da[NC];
    float pr = 0.f, pg = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      sq[j] *= scale;
      const float dkt = bt * su[j];
      dk[j] = -bt * sy[j] + dkt * dt[j];
      ddt[j] = dkt * kk[j] + rt * dd[j];
      pr += dd[j] * dt[j];
      pg += dd[j] * a[j];
      da[j] = g * dd[j];
    }
    const float drt = row16_sum(pr);
    const float dg = row16_sum(pg);
    // the learner's step g = eta beta (1 - beta c)/n, only where n > 0
    float dbt = uw;
    if (n > 0.f) {
      const float dc = -eta * bt * bt / n * dg;
      dbt += eta * (1.f - 2.f * bt * c) / n * dg;
      const float dn = -g / n * dg;
      eta_acc += bt * (1.f - bt * c) / n * dg;
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        ddt[j] += dc * a[j];
        da[j] += dc * dt[j] + dn;
      }
    }
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      dk[j] += 2.f * kk[j] * da[j];
      dd[j] = ddt[j];
    }
    if (rg == 0) {
      store_cols<DK>(gq + tt * DK, cl, sq);
      store_cols<DK>(gk + tt * DK, cl, dk);
    }
    if (threadIdx.x == 0) {
      gbeta[tt] = dbt;
      gr[tt] = drt;
    }
  }
#pragma unroll
  for (int i = 0; i < NR; ++i)
    store_cols<DK>(gS0 + ((size_t)bh * DV + rg + 16 * i) * DK, cl, ds[i]);
  if (rg == 0) store_cols<DK>(gd0 + (size_t)bh * DK, cl, dd);
  if (threadIdx.x == 0) geta[bh] = eta_acc;
}

template <int DK, int DV, typename Tin>
int launch_bwd_t(const BackwardArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  const BwdBufs wb = bwd_bufs(a.ws, BH, a.T, DK, DV);
  const int tk1 = ktimer_before(s, "osdn_bwd_record");
  hipLaunchKernelGGL((osdn_bwd_record_kernel<DK, DV, Tin>), dim3(BH), dim3(kDecThreads), 0, s,
                     a.T, (const Tin*)a.k, (const Tin*)a.v, a.beta, a.r, a.eta, a.d0, a.S0, wb);
  ktimer_after(s, tk1);
  int rc = (int)hipGetLastError();
  if (rc) return rc;
  const int tk2 = ktimer_before(s, "osdn_bwd");
  hipLaunchKernelGGL((osdn_bwd_kernel<DK, DV, Tin>), dim3(BH), dim3(kDecThreads), 0, s, a.T,
                     (const Tin*)a.q, (const Tin*)a.k, a.beta, a.r, a.eta, a.scale,
                     (const Tin*)a.dout, a.dST, a.ddT, wb, a.dq, a.dk, a.dv, a.dbeta, a.dr,
                     a.deta, a.dd0, a.dS0);
  ktimer_after(s, tk2);
  return (int)hipGetLastError();
}

template <int DK, typename Tin>
int launch_bwd_dv(const BackwardArgs& a, hipStream_t s) {
  switch (a.Dv) {
    case 32: return launch_bwd_t<DK, 32, Tin>(a, s);
    case 64: return launch_bwd_t<DK, 64, Tin>(a, s);
    case 128: return launch_bwd_t<DK, 128, Tin>(a, s);
  }
  return -1;
}

template <typename Tin>
int launch_bwd_dk(const BackwardArgs& a, hipStream_t s) {
  switch (a.Dk) {
    case 32: return launch_bwd_dv<32, Tin>(a, s);
    case 64: return launch_bwd_dv<64, Tin>(a, s);
    case 128: return launch_bwd_dv<128, Tin>(a, s);
  }
  return -1;
}

}  // namespace

int launch_backward(const BackwardArgs& a, hipStream_t s) {
  if (a.B * a.H == 0) return 0;
  return a.bf16 ? launch_bwd_dk<__bf16>(a, s) : launch_bwd_dk<float>(a, s);
}

}  // namespace osdn
