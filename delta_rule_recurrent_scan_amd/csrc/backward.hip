// Backward pass of the OSDN forward: the reverse-mode adjoint of the token
// recurrence ([OSDN-it] sections 2.1-2.3), per (batch, head) and token t,
//   a = k_t*k_t, n = ||k_t||^2, c = <d_t, a>, k~ = d_t*k_t,
//   u = v_t - S_{t-1} k_t,  S_t = S_{t-1} + beta_t u k~^T,  o_t = scale S_t q_t,
//   g = eta beta_t (1 - beta_t c)/n (0 when n = 0),  d_{t+1} = r_t d_t + g a.
// Given the adjoints of o, S_T and d_T it produces those of q, k, v, beta, r,
// eta, d0 and S0: the memory update's adjoint and, through k~ and the
// learner's step, the adjoint of the phase-1 preconditioner scan.
//
// The recurrences of S and of its adjoint dS act on each value row on its
// own (row i of S_t needs only row i of S_{t-1}; likewise dS), so a stream's
// rows are split into slices of kBwdSliceRows, one workgroup each, which
// fills the chip with B*H*Dv/32 workgroups. What couples the rows are the
// gradient sums over value rows (S_t^T do, dS^T u, S_{t-1}^T w, u.w) and,
// through dS^T u, the adjoint of the learner; so three kernels:
//   record   (per slice) runs the recurrence forward and stores, per token,
//            the residual u_t of its rows and (one slice) the preconditioner
//            d_t, plus its rows of the state every kCkpt tokens and after
//            the last one (fp32);
//   reverse  (per slice) walks the tokens backwards with its rows of S and
//            dS in registers: S_{t-1} = S_t - beta_t u_t k~_t^T (reset exactly
//            from the stored state every kCkpt tokens), and writes, per
//            token, the slice's share of the four row sums;
//   learner  (one workgroup per stream) walks the tokens backwards once more,
//            adds the slices' shares, and carries the adjoint of d through
//            the learner's step: it forms the gradients of q, k, beta, r and
//            eta, and d0's.
// The state sits in registers in the row layout of row_state.hpp (a row over
// 16 column lanes), with kBwdRG row groups of kBwdNR rows each.
#include "device_common.hpp"
#include "launch.hpp"
#include "bwd_common.hpp"
#include "row_state.hpp"

namespace osdn {

// How far ahead each kernel fetches its token operands (register ring sizes):
// each token's chain step is a few hundred cycles, a fetch from HBM takes
// thousands.
constexpr int kRecAhead = 8, kRevAhead = 4;

size_t backward_workspace_bytes(int B, int H, int T, int Dk, int Dv) {
  const size_t BH = (size_t)B * H;
  const size_t rs = (size_t)Dv / kBwdSliceRows;
  return BH * ((size_t)T * (Dv + Dk) + (size_t)(nckpt(T) + 1) * Dv * Dk +
               (size_t)T * rs * share_width(Dk, false)) * 4;
}

namespace {

struct BwdBufs {
  float *u, *d, *ck, *sh;
};

BwdBufs bwd_bufs(void* ws, int BH, int T, int Dk, int Dv) {
  float* f = static_cast<float*>(ws);
  BwdBufs b;
  b.u = f;
  b.d = b.u + (size_t)BH * T * Dv;
  b.ck = b.d + (size_t)BH * T * Dk;
  b.sh = b.ck + (size_t)BH * (nckpt(T) + 1) * Dv * Dk;
  return b;
}

template <int DK, int DV, typename Tin>
__global__ __launch_bounds__(kBwdThreads) void osdn_bwd_record_kernel(
    int BH, int T, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ beta, const float* __restrict__ r, float eta,
    const float* __restrict__ d0, const float* __restrict__ S0, BwdBufs wb) {
  constexpr int NC = DK / 16, NR = kBwdNR, RS = DV / kBwdSliceRows;
  int bh, sl;
  slice_of(RS, bh, sl);
  if (bh >= BH) return;
  const int cl = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int row0 = sl * kBwdSliceRows + rg;  // rows row0 + kBwdRG i
  const int nck = nckpt(T);
  float* Ub = wb.u + (size_t)bh * T * DV;
  float* Db = wb.d + (size_t)bh * T * DK;
  float* Cb = wb.ck + (size_t)bh * (nck + 1) * DV * DK;

  float s[NR][NC], dv[NC];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    if (S0) {
      load_cols<DK, float>(S0 + ((size_t)bh * DV + row0 + kBwdRG * i) * DK, cl, s[i]);
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

  // token inputs fetched kRecAhead tokens ahead into a ring of register
  // sets (the loop is unrolled by the ring size, so each set is static)
  struct Tok {
    float kk[NC], vv[NR], bt, rt;
  };
  const size_t tb = (size_t)bh * T;
  auto fetch = [&](Tok& o, int t) {
    const size_t tn = tb + t;
    load_cols<DK, Tin>(k + tn * DK, cl, o.kk);
#pragma unroll
    for (int i = 0; i < NR; ++i) o.vv[i] = to_f32(v[tn * DV + row0 + kBwdRG * i]);
    o.bt = beta[tn];
    o.rt = r ? r[tn] : 1.f;
  };
  // (fetches are unconditional, of clamped tokens, so that the compiler can
  // count the loads in flight and waits only for the set it uses)
  Tok ring[kRecAhead];
  if (T > 0) {
#pragma unroll
    for (int u = 0; u < kRecAhead; ++u) fetch(ring[u], min(u, T - 1));
  }
  for (int base = 0; base < T; base += kRecAhead) {
#pragma unroll
    for (int u = 0; u < kRecAhead; ++u) {
      const int t = base + u;
      if (t >= T) break;
      if (t % kCkpt == 0) {
        float* C = Cb + (size_t)(t / kCkpt) * DV * DK;
#pragma unroll
        for (int i = 0; i < NR; ++i) store_cols<DK>(C + (size_t)(row0 + kBwdRG * i) * DK, cl, s[i]);
      }
      const Tok cur = ring[u];
      fetch(ring[u], min(t + kRecAhead, T - 1));
      float n = 0.f, c = 0.f, kt[NC], p[NR];
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const float a = cur.kk[j] * cur.kk[j];
        n += a;
        c += dv[j] * a;
        kt[j] = dv[j] * cur.kk[j];
      }
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < NC; ++j) acc += s[i][j] * cur.kk[j];
        p[i] = acc;
      }
      n = row16_sum(n);
      c = row16_sum(c);
#pragma unroll
      for (int i = 0; i < NR; ++i) p[i] = row16_sum(p[i]);
      if (sl == 0 && rg == 0) store_cols<DK>(Db + (size_t)t * DK, cl, dv);
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const float u0 = cur.vv[i] - p[i];
        Ub[(size_t)t * DV + row0 + kBwdRG * i] = u0;  // the row's 16 lanes agree
        const float bu = cur.bt * u0;
#pragma unroll
        for (int j = 0; j < NC; ++j) s[i][j] += bu * kt[j];
      }
      const float g = n > 0.f ? eta * cur.bt * (1.f - cur.bt * c) / n : 0.f;
#pragma unroll
      for (int j = 0; j < NC; ++j) dv[j] = cur.rt * dv[j] + g * (cur.kk[j] * cur.kk[j]);
    }
  }
  float* C = Cb + (size_t)nck * DV * DK;
#pragma unroll
  for (int i = 0; i < NR; ++i) store_cols<DK>(C + (size_t)(row0 + kBwdRG * i) * DK, cl, s[i]);
}

template <int DK, int DV, typename Tin>
__global__ __launch_bounds__(kBwdThreads) void osdn_bwd_kernel(
    int BH, int T, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const float* __restrict__ beta, float scale, const Tin* __restrict__ dout,
    const float* __restrict__ dST, BwdBufs wb, float* __restrict__ gv,
    float* __restrict__ gS0) {
  constexpr int NC = DK / 16, NR = kBwdNR, RS = DV / kBwdSliceRows;
  constexpr int NW = kBwdThreads / kWave, SW = share_width(DK, false);
  // per-wave row sums of a group of kRevAhead tokens (two groups in turn)
  __shared__ __attribute__((aligned(16))) float red[2][kRevAhead][NW][SW];
  int bh, sl;
  slice_of(RS, bh, sl);
  if (bh >= BH) return;
  const int cl = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int row0 = sl * kBwdSliceRows + rg;
  const int nck = nckpt(T);
  const float* Ub = wb.u + (size_t)bh * T * DV;
  const float* Db = wb.d + (size_t)bh * T * DK;
  const float* Cb = wb.ck + (size_t)bh * (nck + 1) * DV * DK;
  float* Sh = wb.sh + (size_t)bh * T * RS * SW + (size_t)sl * SW;

  // S after the last token and dS, for this slice's rows
  float s[NR][NC], ds[NR][NC];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    load_cols<DK, float>(Cb + (size_t)nck * DV * DK + (size_t)(row0 + kBwdRG * i) * DK, cl, s[i]);
    if (dST) {
      load_cols<DK, float>(dST + ((size_t)bh * DV + row0 + kBwdRG * i) * DK, cl, ds[i]);
    } else {
#pragma unroll
      for (int j = 0; j < NC; ++j) ds[i][j] = 0.f;
    }
  }

  // token inputs fetched kRevAhead tokens ahead into a ring of register
  // sets (the loop is unrolled by the ring size, so each set is static)
  struct Tok {
    float kk[NC], qq[NC], dt[NC], dov[NR], uu[NR], bt;
  };
  const size_t tb = (size_t)bh * T;
  auto fetch = [&](Tok& o, int t) {
    const size_t tt = tb + t;
    load_cols<DK, Tin>(k + tt * DK, cl, o.kk);
    load_cols<DK, Tin>(q + tt * DK, cl, o.qq);
    load_cols<DK, float>(Db + (size_t)t * DK, cl, o.dt);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      o.dov[i] = to_f32(dout[tt * DV + row0 + kBwdRG * i]);
      o.uu[i] = Ub[(size_t)t * DV + row0 + kBwdRG * i];
    }
    o.bt = beta[tt];
  };
  Tok ring[kRevAhead];
  if (T > 0) {
#pragma unroll
    for (int u = 0; u < kRevAhead; ++u) fetch(ring[u], max(T - 1 - u, 0));
  }
  for (int base = 0; base < T; base += kRevAhead) {
    const int b = (base / kRevAhead) & 1;
#pragma unroll
    for (int u = 0; u < kRevAhead; ++u) {
      const int t = T - 1 - (base + u);
      if (t < 0) break;
      const size_t tt = tb + t;
      const Tok cur = ring[u];
      fetch(ring[u], max(t - kRevAhead, 0));
      float kt[NC];
#pragma unroll
      for (int j = 0; j < NC; ++j) kt[j] = cur.dt[j] * cur.kk[j];
      const float* kk = cur.kk;
      const float* qq = cur.qq;
      const float* dov = cur.dov;
      const float* uu = cur.uu;
      const float bt = cur.bt;
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
      if (t % kCkpt == 0) {
        const float* C = Cb + (size_t)(t / kCkpt) * DV * DK;
#pragma unroll
        for (int i = 0; i < NR; ++i) load_cols<DK, float>(C + (size_t)(row0 + kBwdRG * i) * DK, cl, s[i]);
      }
      float pb = 0.f;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
#pragma unroll
        for (int j = 0; j < NC; ++j) py[j] += s[i][j] * w[i];
        pb += uu[i] * w[i];
      }
      pb = cl == 0 ? pb : 0.f;
#pragma unroll
      for (int i = 0; i < NR; ++i)
        if (cl == i) gv[tt * DV + row0 + kBwdRG * i] = bt * w[i];

      // the slice's sums over its rows: four row groups per wave by swaps,
      // the waves through LDS, added up once per group of tokens (below)
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
          red[b][u][wave][col] = pq[j];
          red[b][u][wave][DK + col] = pu[j];
          red[b][u][wave][2 * DK + col] = py[j];
        }
        if (lane == 0) red[b][u][wave][3 * DK] = pb;
      }
    }
    // one barrier per group of tokens (the two groups' buffers alternate),
    // then one coalesced store per token
    __syncthreads();
    const int ng = min(kRevAhead, T - base);
#pragma unroll
    for (int u = 0; u < kRevAhead; ++u) {
      if (u >= ng) break;
      float* sh = Sh + (size_t)(T - 1 - (base + u)) * RS * SW;
      for (int e = threadIdx.x; e < 3 * DK + 1; e += kBwdThreads) {
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < NW; ++m) acc += red[b][u][m][e];
        sh[e] = acc;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NR; ++i)
    store_cols<DK>(gS0 + ((size_t)bh * DV + row0 + kBwdRG * i) * DK, cl, ds[i]);
}

template <int DK, int DV, typename Tin>
int launch_bwd_t(const BackwardArgs& a, hipStream_t s) {
  constexpr int RS = DV / kBwdSliceRows;
  const int BH = a.B * a.H;
  const BwdBufs wb = bwd_bufs(a.ws, BH, a.T, DK, DV);
  const int grid = bwd_grid(BH, RS);
  const int tk1 = ktimer_before(s, "osdn_bwd_record");
  hipLaunchKernelGGL((osdn_bwd_record_kernel<DK, DV, Tin>), dim3(grid), dim3(kBwdThreads), 0, s,
                     BH, a.T, (const Tin*)a.k, (const Tin*)a.v, a.beta, a.r, a.eta, a.d0, a.S0,
                     wb);
  ktimer_after(s, tk1);
  int rc = (int)hipGetLastError();
  if (rc) return rc;
  const int tk2 = ktimer_before(s, "osdn_bwd");
  hipLaunchKernelGGL((osdn_bwd_kernel<DK, DV, Tin>), dim3(grid), dim3(kBwdThreads), 0, s, BH,
                     a.T, (const Tin*)a.q, (const Tin*)a.k, a.beta, a.scale,
                     (const Tin*)a.dout, a.dST, wb, a.dv, a.dS0);
  ktimer_after(s, tk2);
  rc = (int)hipGetLastError();
  if (rc) return rc;
  const int tk3 = ktimer_before(s, "osdn_bwd_learner");
  LearnerArgs la{a.T, a.k, a.beta, a.r, a.eta, a.scale, a.ddT, wb.d, wb.sh,
                 a.dq, a.dk, a.dbeta, a.dr, a.deta, a.dd0, nullptr};
  hipLaunchKernelGGL((osdn_bwd_learner_kernel<DK, DV, Tin, false>), dim3(BH),
                     dim3(kLearnThreads), 0, s, la);
  ktimer_after(s, tk3);
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
