// Gate-aware backward: the reverse-mode adjoints of the two token recurrences
// with a per-key-channel decay,
//   OSDN on a decaying backbone ([OSDN-it] section 4, with the reading that
//   the decay acts on the state before the token's step; state [Dv, Dk]):
//     S_dec = S_{t-1} Diag(alpha_t), u = v - S_dec k, S_t = S_dec + beta u k~^T,
//     d_{t+1} = r d_t + g a as in the plain rule;
//   Gated DeltaNet-2 ([GDN2-it] method, part 1; state [Dk, Dv]):
//     S_dec = Diag(alpha_t) S_{t-1}, u = w*v - S_dec^T (b*k), S_t = S_dec + k u^T,
// both with o_t = scale * (state read with q_t). Both are one rule in the row
// layout of row_state.hpp once GDN-2's state is held transposed (rows =
// value channels, columns = key channels):
//     S_dec = S Diag(alpha), u = y - S_dec x, S_t = S_dec + c u z^T, o = scale S_t q
// with read key x, write key z, target y and coefficient c:
//     OSDN:  x = k,     z = d*k, y = v,     c = beta
//     GDN-2: x = b*k,   z = k,   y = w*v,   c = 1.
// Every reduction over key channels is then a row-of-16 sum, and the sums
// over value channels (the column sums of the adjoint) go through LDS once
// per token.
//
// A decayed state cannot be walked backwards by subtracting the write (that
// would divide by alpha), so the reverse pass recomputes: the state before
// every 64th token is stored by a forward kernel, and the reverse kernel,
// for each 64-token interval from the last, runs the interval forward from
// its stored state writing the state before each token into a per-stream
// buffer, then walks the interval backwards reading them. Each thread reads
// back only the elements it wrote itself.
#include "device_common.hpp"
#include "launch.hpp"
#include "row_state.hpp"

#include <algorithm>

namespace osdn {

constexpr int kGCkpt = 64;  // tokens per recomputed interval

__host__ __device__ inline int gckpt(int T) { return (T + kGCkpt - 1) / kGCkpt; }

size_t gated_backward_workspace_bytes(int B, int H, int T, int Dk, int Dv, int gdn2) {
  const size_t BH = (size_t)B * H;
  const size_t per = (gdn2 ? 0 : (size_t)T * Dk) +
                     (size_t)(gckpt(T) + 1 + std::min(T, kGCkpt)) * Dv * Dk;
  return BH * per * 4;
}

namespace {

struct GBufs {
  float *d, *ck, *sb;  // d: OSDN only
};

GBufs gbufs(void* ws, int BH, int T, int Dk, int Dv, bool g2) {
  float* f = static_cast<float*>(ws);
  GBufs b;
  b.d = f;
  b.ck = b.d + (g2 ? 0 : (size_t)BH * T * Dk);
  b.sb = b.ck + (size_t)BH * (gckpt(T) + 1) * Dv * Dk;
  return b;
}

// One row of a [Dk, Dv] state (GDN-2's memory layout) as the row layout's
// value-channel row m: element (j, m) for each held key channel j.
template <int DK, int DV>
__device__ __forceinline__ void load_colsT(const float* S, int m, int cl, float (&x)[DK / 16]) {
#pragma unroll
  for (int j = 0; j < DK / 16; ++j) x[j] = S[(size_t)dec_col<DK>(cl, j) * DV + m];
}
template <int DK, int DV>
__device__ __forceinline__ void store_colsT(float* S, int m, int cl, const float (&x)[DK / 16]) {
#pragma unroll
  for (int j = 0; j < DK / 16; ++j) S[(size_t)dec_col<DK>(cl, j) * DV + m] = x[j];
}

template <int DK, int DV, bool G2>
__device__ __forceinline__ void load_state(const float* S, int rg, int cl,
                                           float (&s)[DV / 16][DK / 16]) {
#pragma unroll
  for (int i = 0; i < DV / 16; ++i) {
    if constexpr (G2) load_colsT<DK, DV>(S, rg + 16 * i, cl, s[i]);
    else load_cols<DK, float>(S + (size_t)(rg + 16 * i) * DK, cl, s[i]);
  }
}
template <int DK, int DV, bool G2>
__device__ __forceinline__ void store_state(float* S, int rg, int cl,
                                            const float (&s)[DV / 16][DK / 16]) {
#pragma unroll
  for (int i = 0; i < DV / 16; ++i) {
    if constexpr (G2) store_colsT<DK, DV>(S, rg + 16 * i, cl, s[i]);
    else store_cols<DK>(S + (size_t)(rg + 16 * i) * DK, cl, s[i]);
  }
}
// The internal buffers (stored states) are always in the row layout.
template <int DK, int DV>
__device__ __forceinline__ void load_rows(const float* S, int rg, int cl,
                                          float (&s)[DV / 16][DK / 16]) {
#pragma unroll
  for (int i = 0; i < DV / 16; ++i) load_cols<DK, float>(S + (size_t)(rg + 16 * i) * DK, cl, s[i]);
}
template <int DK, int DV>
__device__ __forceinline__ void store_rows(float* S, int rg, int cl,
                                           const float (&s)[DV / 16][DK / 16]) {
#pragma unroll
  for (int i = 0; i < DV / 16; ++i) store_cols<DK>(S + (size_t)(rg + 16 * i) * DK, cl, s[i]);
}

struct GParams {
  int T;
  float eta, scale;
  const void *q, *k, *v, *bg, *wg;  // bg, wg: GDN-2's erase and write gates
  const float *beta, *r, *la, *d0, *S0;
  const void* dout;
  const float *dST, *ddT;
  GBufs wb;
  float *dq, *dk, *dv, *dbeta, *dr, *deta, *dd0, *dS0, *dla, *db, *dw;
};

// One token's operands in the unified form, plus what the OSDN learner needs.
template <int DK, int DV>
struct Tok {
  float kk[DK / 16], x[DK / 16], z[DK / 16], al[DK / 16], y[DV / 16];
  float c;
  float n, cc, bt, rt;  // OSDN: ||k||^2, <d, k*k>, beta, r
};

// A token's inputs as loaded (widened to fp32), before anything that
// depends on the recurrence: loaded one token ahead of their use.
template <int DK, int DV>
struct Raw {
  float kk[DK / 16], la[DK / 16], b[DK / 16], v[DV / 16], w[DV / 16];
  float bt, rt;
};

template <int DK, int DV, typename Tin, bool G2>
__device__ __forceinline__ void raw_load(const GParams& p, size_t tt, int rg, int cl,
                                         Raw<DK, DV>& o) {
  constexpr int NR = DV / 16;
  load_cols<DK, Tin>((const Tin*)p.k + tt * DK, cl, o.kk);
  load_cols<DK, float>(p.la + tt * DK, cl, o.la);
#pragma unroll
  for (int i = 0; i < NR; ++i) o.v[i] = to_f32(((const Tin*)p.v)[tt * DV + rg + 16 * i]);
  if constexpr (G2) {
    load_cols<DK, Tin>((const Tin*)p.bg + tt * DK, cl, o.b);
#pragma unroll
    for (int i = 0; i < NR; ++i) o.w[i] = to_f32(((const Tin*)p.wg)[tt * DV + rg + 16 * i]);
  } else {
    o.bt = p.beta[tt];
    o.rt = p.r ? p.r[tt] : 1.f;
  }
}

// The unified operands x, z, y, c (and OSDN's key statistics) from a token's
// inputs and, for OSDN, its preconditioner dt.
template <int DK, int DV, bool G2>
__device__ __forceinline__ void make_tok(const Raw<DK, DV>& r, const float (&dt)[DK / 16],
                                         Tok<DK, DV>& o) {
  constexpr int NC = DK / 16, NR = DV / 16;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    o.kk[j] = r.kk[j];
    o.al[j] = expf(r.la[j]);
  }
  if constexpr (G2) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      o.x[j] = r.b[j] * r.kk[j];
      o.z[j] = r.kk[j];
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) o.y[i] = r.w[i] * r.v[i];
    o.c = 1.f;
  } else {
    float n = 0.f, c = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const float a = r.kk[j] * r.kk[j];
      n += a;
      c += dt[j] * a;
      o.x[j] = r.kk[j];
      o.z[j] = dt[j] * r.kk[j];
    }
    o.n = row16_sum(n);
    o.cc = row16_sum(c);
#pragma unroll
    for (int i = 0; i < NR; ++i) o.y[i] = r.v[i];
    o.bt = r.bt;
    o.rt = r.rt;
    o.c = r.bt;
  }
}

// s <- S_dec + c u z^T with S_dec = s Diag(alpha), u = y - S_dec x
template <int DK, int DV>
__device__ __forceinline__ void fwd_step(float (&s)[DV / 16][DK / 16], const Tok<DK, DV>& tk) {
  constexpr int NC = DK / 16, NR = DV / 16;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      s[i][j] *= tk.al[j];
      acc += s[i][j] * tk.x[j];
    }
    const float cu = tk.c * (tk.y[i] - row16_sum(acc));
#pragma unroll
    for (int j = 0; j < NC; ++j) s[i][j] += cu * tk.z[j];
  }
}

// OSDN learner step d <- r d + g a
template <int DK, int DV>
__device__ __forceinline__ void learner_step(float (&dv)[DK / 16], const Tok<DK, DV>& tk,
                                             float eta) {
  const float g = tk.n > 0.f ? eta * tk.bt * (1.f - tk.bt * tk.cc) / tk.n : 0.f;
#pragma unroll
  for (int j = 0; j < DK / 16; ++j) dv[j] = tk.rt * dv[j] + g * (tk.kk[j] * tk.kk[j]);
}

template <int DK, int DV, typename Tin, bool G2>
__global__ __launch_bounds__(kDecThreads) void gated_bwd_record_kernel(GParams p) {
  constexpr int NC = DK / 16, NR = DV / 16;
  const int bh = blockIdx.x;
  const int cl = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int T = p.T, nck = gckpt(T);
  float* Db = p.wb.d + (size_t)bh * T * DK;
  float* Cb = p.wb.ck + (size_t)bh * (nck + 1) * DV * DK;

  float s[NR][NC], dv[NC];
  if (p.S0) {
    load_state<DK, DV, G2>(p.S0 + (size_t)bh * DV * DK, rg, cl, s);
  } else {
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int j = 0; j < NC; ++j) s[i][j] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < NC; ++j) dv[j] = 1.f;
  if (!G2 && p.d0) load_cols<DK, float>(p.d0 + (size_t)bh * DK, cl, dv);

  const size_t tb = (size_t)bh * T;
  Raw<DK, DV> nx;
  if (T > 0) raw_load<DK, DV, Tin, G2>(p, tb, rg, cl, nx);
  for (int t = 0; t < T; ++t) {
    if (t % kGCkpt == 0) store_rows<DK, DV>(Cb + (size_t)(t / kGCkpt) * DV * DK, rg, cl, s);
    if (!G2 && rg == 0) store_cols<DK>(Db + (size_t)t * DK, cl, dv);
    const Raw<DK, DV> cur = nx;
    if (t + 1 < T) raw_load<DK, DV, Tin, G2>(p, tb + t + 1, rg, cl, nx);
    Tok<DK, DV> tk;
    make_tok<DK, DV, G2>(cur, dv, tk);
    fwd_step<DK, DV>(s, tk);
    if constexpr (!G2) learner_step<DK, DV>(dv, tk, p.eta);
  }
  store_rows<DK, DV>(Cb + (size_t)nck * DV * DK, rg, cl, s);
}

template <int DK, int DV, typename Tin, bool G2>
__global__ __launch_bounds__(kDecThreads) void gated_bwd_kernel(GParams p) {
  constexpr int NC = DK / 16, NR = DV / 16, NW = kDecThreads / kWave;
  // per wave: S_dec^T do, dS^T u, S_dec^T (c w), colsum(dS_dec * S_dec),
  // then u.do and u.w
  constexpr int RW = 4 * DK + 4;
  __shared__ float red[2][NW][RW];
  const int bh = blockIdx.x;
  const int cl = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int T = p.T, nck = gckpt(T);
  const float* Db = p.wb.d + (size_t)bh * T * DK;
  const float* Cb = p.wb.ck + (size_t)bh * (nck + 1) * DV * DK;
  float* Sb = p.wb.sb + (size_t)bh * min(T, kGCkpt) * DV * DK;
  const Tin* q = (const Tin*)p.q;
  const Tin* dout = (const Tin*)p.dout;

  float s[NR][NC], ds[NR][NC], dd[NC];
  if (p.dST) {
    load_state<DK, DV, G2>(p.dST + (size_t)bh * DV * DK, rg, cl, ds);
  } else {
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int j = 0; j < NC; ++j) ds[i][j] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < NC; ++j) dd[j] = 0.f;
  if (!G2 && p.ddT) load_cols<DK, float>(p.ddT + (size_t)bh * DK, cl, dd);
  float eta_acc = 0.f;
  int par = 0;

  const size_t tb = (size_t)bh * T;
  for (int iv = nck - 1; iv >= 0; --iv) {
    const int t0 = iv * kGCkpt, t1 = min(T, t0 + kGCkpt) - 1;
    // the interval forward: the state before each of its tokens but the last
    // (inputs one token ahead)
    load_rows<DK, DV>(Cb + (size_t)iv * DV * DK, rg, cl, s);
    Raw<DK, DV> nx;
    float dn[NC];
    if (t0 < t1) {
      raw_load<DK, DV, Tin, G2>(p, tb + t0, rg, cl, nx);
      if constexpr (!G2) load_cols<DK, float>(Db + (size_t)t0 * DK, cl, dn);
    }
    for (int t = t0; t < t1; ++t) {
      store_rows<DK, DV>(Sb + (size_t)(t - t0) * DV * DK, rg, cl, s);
      const Raw<DK, DV> cur = nx;
      float dt[NC];
#pragma unroll
      for (int j = 0; j < NC; ++j) dt[j] = dn[j];
      if (t + 1 < t1) {
        raw_load<DK, DV, Tin, G2>(p, tb + t + 1, rg, cl, nx);
        if constexpr (!G2) load_cols<DK, float>(Db + (size_t)(t + 1) * DK, cl, dn);
      }
      Tok<DK, DV> tk;
      make_tok<DK, DV, G2>(cur, dt, tk);
      fwd_step<DK, DV>(s, tk);
    }
    // and backwards through it (inputs one token ahead)
    float qn[NC], don[NR];
    auto prefetch = [&](int t) {
      const size_t tt = tb + t;
      raw_load<DK, DV, Tin, G2>(p, tt, rg, cl, nx);
      if constexpr (!G2) load_cols<DK, float>(Db + (size_t)t * DK, cl, dn);
      load_cols<DK, Tin>(q + tt * DK, cl, qn);
#pragma unroll
      for (int i = 0; i < NR; ++i) don[i] = to_f32(dout[tt * DV + rg + 16 * i]);
    };
    prefetch(t1);
    for (int t = t1; t >= t0; --t) {
      if (t < t1) load_rows<DK, DV>(Sb + (size_t)(t - t0) * DV * DK, rg, cl, s);
      const size_t tt = tb + t;
      float dt[NC], qq[NC], dov[NR];
      const Raw<DK, DV> cur = nx;
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        dt[j] = dn[j];
        qq[j] = qn[j];
      }
#pragma unroll
      for (int i = 0; i < NR; ++i) dov[i] = don[i];
      if (t > t0) prefetch(t - 1);
      Tok<DK, DV> tk;
      make_tok<DK, DV, G2>(cur, dt, tk);

      // S_dec, u = y - S_dec x; dS += scale do q^T; w = dS z (row sums)
      float u[NR], w[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        float acc = 0.f, acw = 0.f;
        const float sd = p.scale * dov[i];
#pragma unroll
        for (int j = 0; j < NC; ++j) {
          s[i][j] *= tk.al[j];
          acc += s[i][j] * tk.x[j];
          ds[i][j] += sd * qq[j];
          acw += ds[i][j] * tk.z[j];
        }
        u[i] = acc;
        w[i] = acw;
      }
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        u[i] = tk.y[i] - row16_sum(u[i]);
        w[i] = row16_sum(w[i]);
      }
      // column partials; the adjoint of u is c w; dS_dec = dS - c w x^T;
      // dS_{t-1} = dS_dec Diag(alpha)
      float pq[NC], pu[NC], py[NC], pa[NC], ud = 0.f, uw = 0.f;
#pragma unroll
      for (int j = 0; j < NC; ++j) pq[j] = pu[j] = py[j] = pa[j] = 0.f;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const float cw = tk.c * w[i];
        ud += u[i] * dov[i];
        uw += u[i] * w[i];
#pragma unroll
        for (int j = 0; j < NC; ++j) {
          pq[j] += s[i][j] * dov[i];
          pu[j] += ds[i][j] * u[i];
          py[j] += s[i][j] * cw;
          const float dsd = ds[i][j] - cw * tk.x[j];
          pa[j] += dsd * s[i][j];
          ds[i][j] = dsd * tk.al[j];
        }
      }
      ud = cl == 0 ? ud : 0.f;
      uw = cl == 0 ? uw : 0.f;
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        pq[j] = add_swap32(add_swap16(pq[j]));
        pu[j] = add_swap32(add_swap16(pu[j]));
        py[j] = add_swap32(add_swap16(py[j]));
        pa[j] = add_swap32(add_swap16(pa[j]));
      }
      ud = wave_sum(ud);
      uw = wave_sum(uw);
      const int b = par;
      par ^= 1;
      if (lane < 16) {
#pragma unroll
        for (int j = 0; j < NC; ++j) {
          const int col = dec_col<DK>(cl, j);
          red[b][wave][col] = pq[j];
          red[b][wave][DK + col] = pu[j];
          red[b][wave][2 * DK + col] = py[j];
          red[b][wave][3 * DK + col] = pa[j];
        }
        if (lane == 0) {
          red[b][wave][4 * DK] = ud;
          red[b][wave][4 * DK + 1] = uw;
        }
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const int col = dec_col<DK>(cl, j);
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
        for (int m = 0; m < NW; ++m) {
          a0 += red[b][m][col];
          a1 += red[b][m][DK + col];
          a2 += red[b][m][2 * DK + col];
          a3 += red[b][m][3 * DK + col];
        }
        pq[j] = a0;
        pu[j] = a1;
        py[j] = a2;
        pa[j] = a3;
      }
      ud = uw = 0.f;
#pragma unroll
      for (int m = 0; m < NW; ++m) {
        ud += red[b][m][4 * DK];
        uw += red[b][m][4 * DK + 1];
      }

      // S_t^T do = S_dec^T do + c z (u.do); the adjoints of z (c dS^T u),
      // of x (-S_dec^T (c w)) and of log alpha
      float gq[NC], gx[NC], gz[NC];
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        gq[j] = p.scale * (pq[j] + tk.c * tk.z[j] * ud);
        gz[j] = tk.c * pu[j];
        gx[j] = -py[j];
      }
      if (rg == 0) {
        store_cols<DK>(p.dq + tt * DK, cl, gq);
        store_cols<DK>(p.dla + tt * DK, cl, pa);
      }
      if constexpr (G2) {
        // x = b*k, z = k, y = w*v
        float gk[NC], gb[NC];
#pragma unroll
        for (int j = 0; j < NC; ++j) {
          gk[j] = gz[j] + cur.b[j] * gx[j];
          gb[j] = tk.kk[j] * gx[j];
        }
        if (rg == 0) {
          store_cols<DK>(p.dk + tt * DK, cl, gk);
          store_cols<DK>(p.db + tt * DK, cl, gb);
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          if (cl == (i & 15)) {
            const size_t e = tt * DV + rg + 16 * i;
            p.dv[e] = cur.w[i] * w[i];
            p.dw[e] = cur.v[i] * w[i];
          }
        }
      } else {
        // x = k, z = d*k, y = v, c = beta; then the learner's adjoint
#pragma unroll
        for (int i = 0; i < NR; ++i)
          if (cl == (i & 15)) p.dv[tt * DV + rg + 16 * i] = tk.bt * w[i];
        float dk[NC], ddt[NC], da[NC];
        float pr = 0.f, pg = 0.f;
#pragma unroll
        for (int j = 0; j < NC; ++j) {
          const float a = tk.kk[j] * tk.kk[j];
          dk[j] = gx[j] + gz[j] * dt[j];
          ddt[j] = gz[j] * tk.kk[j] + tk.rt * dd[j];
          pr += dd[j] * dt[j];
          pg += dd[j] * a;
        }
        const float drt = row16_sum(pr);
        const float dg = row16_sum(pg);
        const float g = tk.n > 0.f ? p.eta * tk.bt * (1.f - tk.bt * tk.cc) / tk.n : 0.f;
#pragma unroll
        for (int j = 0; j < NC; ++j) da[j] = g * dd[j];
        float dbt = uw;
        if (tk.n > 0.f) {
          const float dc = -p.eta * tk.bt * tk.bt / tk.n * dg;
          dbt += p.eta * (1.f - 2.f * tk.bt * tk.cc) / tk.n * dg;
          const float dn = -g / tk.n * dg;
          eta_acc += tk.bt * (1.f - tk.bt * tk.cc) / tk.n * dg;
#pragma unroll
          for (int j = 0; j < NC; ++j) {
            const float a = tk.kk[j] * tk.kk[j];
            ddt[j] += dc * a;
            da[j] += dc * dt[j] + dn;
          }
        }
#pragma unroll
        for (int j = 0; j < NC; ++j) {
          dk[j] += 2.f * tk.kk[j] * da[j];
          dd[j] = ddt[j];
        }
        if (rg == 0) store_cols<DK>(p.dk + tt * DK, cl, dk);
        if (threadIdx.x == 0) {
          p.dbeta[tt] = dbt;
          p.dr[tt] = drt;
        }
      }
    }
  }
  store_state<DK, DV, G2>(p.dS0 + (size_t)bh * DV * DK, rg, cl, ds);
  if constexpr (!G2) {
    if (rg == 0) store_cols<DK>(p.dd0 + (size_t)bh * DK, cl, dd);
    if (threadIdx.x == 0) p.deta[bh] = eta_acc;
  }
}

template <int DK, int DV, typename Tin, bool G2>
int launch_gbwd_t(const GatedBackwardArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  GParams p{a.T, a.eta, a.scale, a.q, a.k, a.v, a.b, a.w, a.beta, a.r, a.log_alpha,
            a.d0, a.S0, a.dout, a.dST, a.ddT, gbufs(a.ws, BH, a.T, DK, DV, G2),
            a.dq, a.dk, a.dv, a.dbeta, a.dr, a.deta, a.dd0, a.dS0, a.dla, a.db, a.dw};
  const int tk1 = ktimer_before(s, G2 ? "gdn2_bwd_record" : "gated_bwd_record");
  hipLaunchKernelGGL((gated_bwd_record_kernel<DK, DV, Tin, G2>), dim3(BH), dim3(kDecThreads),
                     0, s, p);
  ktimer_after(s, tk1);
  int rc = (int)hipGetLastError();
  if (rc) return rc;
  const int tk2 = ktimer_before(s, G2 ? "gdn2_bwd" : "gated_bwd");
  hipLaunchKernelGGL((gated_bwd_kernel<DK, DV, Tin, G2>), dim3(BH), dim3(kDecThreads), 0, s, p);
  ktimer_after(s, tk2);
  return (int)hipGetLastError();
}

template <int DK, typename Tin, bool G2>
int launch_gbwd_dv(const GatedBackwardArgs& a, hipStream_t s) {
  switch (a.Dv) {
    case 32: return launch_gbwd_t<DK, 32, Tin, G2>(a, s);
    case 64: return launch_gbwd_t<DK, 64, Tin, G2>(a, s);
    case 128: return launch_gbwd_t<DK, 128, Tin, G2>(a, s);
  }
  return -1;
}

template <typename Tin, bool G2>
int launch_gbwd_dk(const GatedBackwardArgs& a, hipStream_t s) {
  switch (a.Dk) {
    case 32: return launch_gbwd_dv<32, Tin, G2>(a, s);
    case 64: return launch_gbwd_dv<64, Tin, G2>(a, s);
    case 128: return launch_gbwd_dv<128, Tin, G2>(a, s);
  }
  return -1;
}

}  // namespace

int launch_gated_backward(const GatedBackwardArgs& a, hipStream_t s) {
  if (a.B * a.H == 0) return 0;
  if (a.gdn2)
    return a.bf16 ? launch_gbwd_dk<__bf16, true>(a, s) : launch_gbwd_dk<float, true>(a, s);
  return a.bf16 ? launch_gbwd_dk<__bf16, false>(a, s) : launch_gbwd_dk<float, false>(a, s);
}

}  // namespace osdn
