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
// The S and dS recurrences act on each value row on its own, so as for the
// plain rule a stream's rows are split into 32-row slices, one workgroup
// each (bwd_common.hpp); per token each slice writes its sums over its rows
// of S_dec^T do, dS^T u, S_dec^T w, u.w, u.do and dS_dec * S_dec, and a last
// kernel adds them: for OSDN the learner of bwd_common.hpp (which also
// carries the preconditioner's adjoint), for GDN-2 a token-parallel kernel.
//
// A decayed state cannot be walked backwards by subtracting the write (that
// would divide by alpha), so the reverse pass recomputes: the state before
// every 64th token is stored by a forward kernel, and the reverse kernel,
// for each 64-token interval from the last, runs the interval forward from
// its stored state writing the state before each token into a per-slice
// buffer, then walks the interval backwards reading them. Each thread reads
// back only the elements it wrote itself.
#include "bwd_common.hpp"
#include "device_common.hpp"
#include "launch.hpp"
#include "row_state.hpp"

#include <algorithm>

namespace osdn {

constexpr int kGRecAhead = 8, kGRevAhead = 4;  // token-operand fetch distances

size_t gated_backward_workspace_bytes(int B, int H, int T, int Dk, int Dv, int gdn2) {
  const size_t BH = (size_t)B * H;
  const size_t rs = (size_t)Dv / kBwdSliceRows;
  const size_t per = (gdn2 ? 0 : (size_t)T * Dk) +
                     (size_t)(nckpt(T) + 1 + std::min(T, kCkpt)) * Dv * Dk +
                     (size_t)T * rs * share_width(Dk, true);
  return BH * per * 4;
}

namespace {

struct GBufs {
  float *d, *ck, *sb, *sh;  // d: OSDN only
};

GBufs gbufs(void* ws, int BH, int T, int Dk, int Dv, bool g2) {
  float* f = static_cast<float*>(ws);
  GBufs b;
  b.d = f;
  b.ck = b.d + (g2 ? 0 : (size_t)BH * T * Dk);
  b.sb = b.ck + (size_t)BH * (nckpt(T) + 1) * Dv * Dk;
  b.sh = b.sb + (size_t)BH * std::min(T, kCkpt) * Dv * Dk;
  return b;
}

// Value row m of a state as the row layout holds it: OSDN's [Dv, Dk] row m,
// or (G2) column m of GDN-2's [Dk, Dv].
template <int DK, int DV, bool G2>
__device__ __forceinline__ void load_state_row(const float* S, int m, int cl,
                                               float (&x)[DK / 16]) {
  if constexpr (G2) {
#pragma unroll
    for (int j = 0; j < DK / 16; ++j) x[j] = S[(size_t)dec_col<DK>(cl, j) * DV + m];
  } else {
    load_cols<DK, float>(S + (size_t)m * DK, cl, x);
  }
}
template <int DK, int DV, bool G2>
__device__ __forceinline__ void store_state_row(float* S, int m, int cl,
                                                const float (&x)[DK / 16]) {
  if constexpr (G2) {
#pragma unroll
    for (int j = 0; j < DK / 16; ++j) S[(size_t)dec_col<DK>(cl, j) * DV + m] = x[j];
  } else {
    store_cols<DK>(S + (size_t)m * DK, cl, x);
  }
}

struct GParams {
  int BH, T;
  float eta, scale;
  const void *q, *k, *v, *bg, *wg;  // bg, wg: GDN-2's erase and write gates
  const float *beta, *r, *la, *d0, *S0;
  const void* dout;
  const float* dST;
  GBufs wb;
  float *dv, *dw, *dS0;
};

// A token's inputs as loaded (widened to fp32) for this thread's rows and
// channels, before anything that depends on the recurrence.
template <int DK>
struct Raw {
  float kk[DK / 16], al[DK / 16], b[DK / 16], v[kBwdNR], w[kBwdNR];
  float bt, rt;
};

template <int DK, int DV, typename Tin, bool G2>
__device__ __forceinline__ void raw_load(const GParams& p, size_t tt, int row0, int cl,
                                         Raw<DK>& o) {
  load_cols<DK, Tin>((const Tin*)p.k + tt * DK, cl, o.kk);
  load_cols<DK, float>(p.la + tt * DK, cl, o.al);
#pragma unroll
  for (int i = 0; i < kBwdNR; ++i)
    o.v[i] = to_f32(((const Tin*)p.v)[tt * DV + row0 + kBwdRG * i]);
  if constexpr (G2) {
    load_cols<DK, Tin>((const Tin*)p.bg + tt * DK, cl, o.b);
#pragma unroll
    for (int i = 0; i < kBwdNR; ++i)
      o.w[i] = to_f32(((const Tin*)p.wg)[tt * DV + row0 + kBwdRG * i]);
  } else {
    o.bt = p.beta[tt];
    o.rt = p.r ? p.r[tt] : 1.f;
  }
}

// The unified operands from a token's inputs and, for OSDN, its
// preconditioner dt: decay factors, read key x, write key z, target y,
// coefficient c (and OSDN's key statistics).
template <int DK>
struct Tok {
  float kk[DK / 16], al[DK / 16], x[DK / 16], z[DK / 16], y[kBwdNR];
  float c, n, cc, bt, rt;
};

template <int DK, bool G2>
__device__ __forceinline__ void make_tok(const Raw<DK>& r, const float (&dt)[DK / 16],
                                         Tok<DK>& o) {
  constexpr int NC = DK / 16;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    o.kk[j] = r.kk[j];
    o.al[j] = expf(r.al[j]);
  }
  if constexpr (G2) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      o.x[j] = r.b[j] * r.kk[j];
      o.z[j] = r.kk[j];
    }
#pragma unroll
    for (int i = 0; i < kBwdNR; ++i) o.y[i] = r.w[i] * r.v[i];
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
    for (int i = 0; i < kBwdNR; ++i) o.y[i] = r.v[i];
    o.bt = r.bt;
    o.rt = r.rt;
    o.c = r.bt;
  }
}

// s <- S_dec + c u z^T with S_dec = s Diag(alpha), u = y - S_dec x
template <int DK>
__device__ __forceinline__ void fwd_step(float (&s)[kBwdNR][DK / 16], const Tok<DK>& tk) {
  constexpr int NC = DK / 16;
#pragma unroll
  for (int i = 0; i < kBwdNR; ++i) {
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

template <int DK, int DV, typename Tin, bool G2>
__global__ __launch_bounds__(kBwdThreads) void gated_bwd_record_kernel(GParams p) {
  constexpr int NC = DK / 16, NR = kBwdNR, RS = DV / kBwdSliceRows;
  int bh, sl;
  slice_of(RS, bh, sl);
  if (bh >= p.BH) return;
  const int cl = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int row0 = sl * kBwdSliceRows + rg;  // rows row0 + kBwdRG i
  const int T = p.T, nck = nckpt(T);
  float* Db = p.wb.d + (size_t)bh * T * DK;
  float* Cb = p.wb.ck + (size_t)bh * (nck + 1) * DV * DK;

  float s[NR][NC], dv[NC];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    if (p.S0) {
      load_state_row<DK, DV, G2>(p.S0 + (size_t)bh * DV * DK, row0 + kBwdRG * i, cl, s[i]);
    } else {
#pragma unroll
      for (int j = 0; j < NC; ++j) s[i][j] = 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < NC; ++j) dv[j] = 1.f;
  if (!G2 && p.d0) load_cols<DK, float>(p.d0 + (size_t)bh * DK, cl, dv);

  // token inputs fetched kGRecAhead tokens ahead into a ring of register
  // sets: unconditional fetches of clamped tokens, the loop unrolled by the
  // ring size so that each set is static
  const size_t tb = (size_t)bh * T;
  Raw<DK> ring[kGRecAhead];
  if (T > 0) {
#pragma unroll
    for (int u = 0; u < kGRecAhead; ++u)
      raw_load<DK, DV, Tin, G2>(p, tb + min(u, T - 1), row0, cl, ring[u]);
  }
  for (int base = 0; base < T; base += kGRecAhead) {
#pragma unroll
    for (int u = 0; u < kGRecAhead; ++u) {
      const int t = base + u;
      if (t >= T) break;
      if (t % kCkpt == 0) {
        float* C = Cb + (size_t)(t / kCkpt) * DV * DK;
#pragma unroll
        for (int i = 0; i < NR; ++i)
          store_cols<DK>(C + (size_t)(row0 + kBwdRG * i) * DK, cl, s[i]);
      }
      if (!G2 && sl == 0 && rg == 0) store_cols<DK>(Db + (size_t)t * DK, cl, dv);
      const Raw<DK> cur = ring[u];
      raw_load<DK, DV, Tin, G2>(p, tb + min(t + kGRecAhead, T - 1), row0, cl, ring[u]);
      Tok<DK> tk;
      make_tok<DK, G2>(cur, dv, tk);
      fwd_step<DK>(s, tk);
      if constexpr (!G2) {
        const float g = tk.n > 0.f ? p.eta * tk.bt * (1.f - tk.bt * tk.cc) / tk.n : 0.f;
#pragma unroll
        for (int j = 0; j < NC; ++j) dv[j] = tk.rt * dv[j] + g * (tk.kk[j] * tk.kk[j]);
      }
    }
  }
  float* C = Cb + (size_t)nck * DV * DK;
#pragma unroll
  for (int i = 0; i < NR; ++i) store_cols<DK>(C + (size_t)(row0 + kBwdRG * i) * DK, cl, s[i]);
}

template <int DK, int DV, typename Tin, bool G2>
__global__ __launch_bounds__(kBwdThreads) void gated_bwd_kernel(GParams p) {
  constexpr int NC = DK / 16, NR = kBwdNR, RS = DV / kBwdSliceRows;
  constexpr int NW = kBwdThreads / kWave, SW = share_width(DK, true);
  // per wave: S_dec^T do, dS^T u, S_dec^T w, then u.w, u.do (pad), then the
  // column sums of dS_dec * S_dec
  // per-wave row sums of a group of kGRevAhead tokens (two groups in turn)
  __shared__ __attribute__((aligned(16))) float red[2][kGRevAhead][NW][SW];
  int grp = 0;  // groups so far (their buffers alternate across intervals)
  int bh, sl;
  slice_of(RS, bh, sl);
  if (bh >= p.BH) return;
  const int cl = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int row0 = sl * kBwdSliceRows + rg;
  const int T = p.T, nck = nckpt(T), LI = min(T, kCkpt);
  const float* Db = p.wb.d + (size_t)bh * T * DK;
  const float* Cb = p.wb.ck + (size_t)bh * (nck + 1) * DV * DK;
  // this slice's rows of the states before each token of an interval
  float* Sb = p.wb.sb + (size_t)bh * LI * DV * DK + (size_t)sl * kBwdSliceRows * DK;
  float* Shb = p.wb.sh + (size_t)bh * T * RS * SW + (size_t)sl * SW;
  const Tin* q = (const Tin*)p.q;
  const Tin* dout = (const Tin*)p.dout;
  const size_t tb = (size_t)bh * T;
  auto sb_row = [&](int t, int i) {
    return Sb + (size_t)t * DV * DK + (size_t)(rg + kBwdRG * i) * DK;
  };

  float s[NR][NC], ds[NR][NC];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    if (p.dST) {
      load_state_row<DK, DV, G2>(p.dST + (size_t)bh * DV * DK, row0 + kBwdRG * i, cl, ds[i]);
    } else {
#pragma unroll
      for (int j = 0; j < NC; ++j) ds[i][j] = 0.f;
    }
  }

  // the reverse walk's token operands: inputs, d_t (OSDN), q and do
  struct RTok {
    Raw<DK> raw;
    float dt[NC], qq[NC], dov[NR];
  };
  auto rfetch = [&](RTok& o, int t) {
    const size_t tt = tb + t;
    raw_load<DK, DV, Tin, G2>(p, tt, row0, cl, o.raw);
    if constexpr (!G2) load_cols<DK, float>(Db + (size_t)t * DK, cl, o.dt);
    load_cols<DK, Tin>(q + tt * DK, cl, o.qq);
#pragma unroll
    for (int i = 0; i < NR; ++i) o.dov[i] = to_f32(dout[tt * DV + row0 + kBwdRG * i]);
  };

  for (int iv = nck - 1; iv >= 0; --iv) {
    const int t0 = iv * kCkpt, t1 = min(T, t0 + kCkpt) - 1;
    // the interval forward: the state before each of its tokens but the last
#pragma unroll
    for (int i = 0; i < NR; ++i)
      load_cols<DK, float>(Cb + (size_t)iv * DV * DK + (size_t)(row0 + kBwdRG * i) * DK, cl,
                           s[i]);
    {
      RTok fr[kGRevAhead];
#pragma unroll
      for (int u = 0; u < kGRevAhead; ++u) rfetch(fr[u], min(t0 + u, t1));
      for (int base = t0; base < t1; base += kGRevAhead) {
#pragma unroll
        for (int u = 0; u < kGRevAhead; ++u) {
          const int t = base + u;
          if (t >= t1) break;
#pragma unroll
          for (int i = 0; i < NR; ++i) store_cols<DK>(sb_row(t - t0, i), cl, s[i]);
          const RTok cur = fr[u];
          rfetch(fr[u], min(t + kGRevAhead, t1));
          Tok<DK> tk;
          make_tok<DK, G2>(cur.raw, cur.dt, tk);
          fwd_step<DK>(s, tk);
        }
      }
    }
    // and backwards through it; the state before each token is fetched one
    // token ahead (the state before the last token is still in s)
    RTok ring[kGRevAhead];
#pragma unroll
    for (int u = 0; u < kGRevAhead; ++u) rfetch(ring[u], max(t1 - u, t0));
    float sn[NR][NC];
#pragma unroll
    for (int i = 0; i < NR; ++i) load_cols<DK, float>(sb_row(max(t1 - 1, t0) - t0, i), cl, sn[i]);
    for (int base = 0; base <= t1 - t0; base += kGRevAhead, ++grp) {
      const int b = grp & 1;
#pragma unroll
      for (int u = 0; u < kGRevAhead; ++u) {
        const int t = t1 - (base + u);
        if (t < t0) break;
        if (t < t1) {
#pragma unroll
          for (int i = 0; i < NR; ++i) {
#pragma unroll
            for (int j = 0; j < NC; ++j) s[i][j] = sn[i][j];
          }
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) load_cols<DK, float>(sb_row(max(t - 1, t0) - t0, i), cl, sn[i]);
        const size_t tt = tb + t;
        const RTok cur = ring[u];
        rfetch(ring[u], max(t - kGRevAhead, t0));
        Tok<DK> tk;
        make_tok<DK, G2>(cur.raw, cur.dt, tk);

        // S_dec, u = y - S_dec x; dS += scale do q^T; w = dS z (row sums)
        float u0[NR], w[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          float acc = 0.f, acw = 0.f;
          const float sd = p.scale * cur.dov[i];
#pragma unroll
          for (int j = 0; j < NC; ++j) {
            s[i][j] *= tk.al[j];
            acc += s[i][j] * tk.x[j];
            ds[i][j] += sd * cur.qq[j];
            acw += ds[i][j] * tk.z[j];
          }
          u0[i] = acc;
          w[i] = acw;
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          u0[i] = tk.y[i] - row16_sum(u0[i]);
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
          ud += u0[i] * cur.dov[i];
          uw += u0[i] * w[i];
#pragma unroll
          for (int j = 0; j < NC; ++j) {
            pq[j] += s[i][j] * cur.dov[i];
            pu[j] += ds[i][j] * u0[i];
            py[j] += s[i][j] * w[i];
            const float dsd = ds[i][j] - cw * tk.x[j];
            pa[j] += dsd * s[i][j];
            ds[i][j] = dsd * tk.al[j];
          }
        }
        // the rows' own gradients: OSDN dv = beta w; GDN-2 dv = w_gate * w,
        // dw = v * w
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          if (cl == i) {
            const size_t e = tt * DV + row0 + kBwdRG * i;
            if constexpr (G2) {
              p.dv[e] = cur.raw.w[i] * w[i];
              p.dw[e] = cur.raw.v[i] * w[i];
            } else {
              p.dv[e] = tk.bt * w[i];
            }
          }
        }
        ud = cl == 0 ? ud : 0.f;
        uw = cl == 0 ? uw : 0.f;
        // the slice's sums over its rows: four row groups per wave by
        // swaps, the waves through LDS, added up once per group of tokens
        // (below)
#pragma unroll
        for (int j = 0; j < NC; ++j) {
          pq[j] = add_swap32(add_swap16(pq[j]));
          pu[j] = add_swap32(add_swap16(pu[j]));
          py[j] = add_swap32(add_swap16(py[j]));
          pa[j] = add_swap32(add_swap16(pa[j]));
        }
        ud = wave_sum(ud);
        uw = wave_sum(uw);
        if (lane < 16) {
#pragma unroll
          for (int j = 0; j < NC; ++j) {
            const int col = dec_col<DK>(cl, j);
            red[b][u][wave][col] = pq[j];
            red[b][u][wave][DK + col] = pu[j];
            red[b][u][wave][2 * DK + col] = py[j];
            red[b][u][wave][3 * DK + 4 + col] = pa[j];
          }
          if (lane == 0) {
            red[b][u][wave][3 * DK] = uw;
            red[b][u][wave][3 * DK + 1] = ud;
          }
        }
      }
      // one barrier per group of tokens, then one coalesced store per token
      __syncthreads();
      const int ng = min(kGRevAhead, t1 - t0 + 1 - base);
#pragma unroll
      for (int u = 0; u < kGRevAhead; ++u) {
        if (u >= ng) break;
        float* sh = Shb + (size_t)(t1 - (base + u)) * RS * SW;
        for (int e = threadIdx.x; e < SW; e += kBwdThreads) {
          float acc = 0.f;
#pragma unroll
          for (int m = 0; m < NW; ++m) acc += red[b][u][m][e];
          sh[e] = acc;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NR; ++i)
    store_state_row<DK, DV, G2>(p.dS0 + (size_t)bh * DV * DK, row0 + kBwdRG * i, cl, ds[i]);
}

// GDN-2's per-token gradients from the slices' sums (no chain): with x = b*k,
// z = k, c = 1: dq = scale (S_dec^T do + k (u.do)), dz = dS^T u,
// dx = -S_dec^T w, dk = dz + b dx, db = k dx, dlog alpha = the decay sums.
// One thread per (token, four channels).
template <int DK, int DV, typename Tin>
__global__ __launch_bounds__(256) void gdn2_bwd_out_kernel(
    int BH, int T, const Tin* __restrict__ k, const Tin* __restrict__ bg, float scale,
    const float* __restrict__ shares, float* __restrict__ gq, float* __restrict__ gk,
    float* __restrict__ gb, float* __restrict__ gla) {
  constexpr int RS = DV / kBwdSliceRows, SW = share_width(DK, true), NQ = DK / 4;
  const size_t item = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (item >= (size_t)BH * T * NQ) return;
  const size_t tt = item / NQ;
  const int c0 = 4 * (int)(item - tt * NQ);
  const float* sh = shares + tt * RS * SW;
  float sq[4] = {0.f, 0.f, 0.f, 0.f}, su[4] = {0.f, 0.f, 0.f, 0.f};
  float sy[4] = {0.f, 0.f, 0.f, 0.f}, sa[4] = {0.f, 0.f, 0.f, 0.f};
  float ud = 0.f;
#pragma unroll
  for (int sl = 0; sl < RS; ++sl) {
    const float* x = sh + sl * SW;
    const float4 a = *reinterpret_cast<const float4*>(x + c0);
    const float4 b = *reinterpret_cast<const float4*>(x + DK + c0);
    const float4 c = *reinterpret_cast<const float4*>(x + 2 * DK + c0);
    const float4 d = *reinterpret_cast<const float4*>(x + 3 * DK + 4 + c0);
    sq[0] += a.x; sq[1] += a.y; sq[2] += a.z; sq[3] += a.w;
    su[0] += b.x; su[1] += b.y; su[2] += b.z; su[3] += b.w;
    sy[0] += c.x; sy[1] += c.y; sy[2] += c.z; sy[3] += c.w;
    sa[0] += d.x; sa[1] += d.y; sa[2] += d.z; sa[3] += d.w;
    ud += x[3 * DK + 1];
  }
  float oq[4], ok[4], ob[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float kv = to_f32(k[tt * DK + c0 + e]), bv = to_f32(bg[tt * DK + c0 + e]);
    const float dx = -sy[e];
    oq[e] = scale * (sq[e] + kv * ud);
    ok[e] = su[e] + bv * dx;
    ob[e] = kv * dx;
  }
  *reinterpret_cast<float4*>(gq + tt * DK + c0) = float4{oq[0], oq[1], oq[2], oq[3]};
  *reinterpret_cast<float4*>(gk + tt * DK + c0) = float4{ok[0], ok[1], ok[2], ok[3]};
  *reinterpret_cast<float4*>(gb + tt * DK + c0) = float4{ob[0], ob[1], ob[2], ob[3]};
  *reinterpret_cast<float4*>(gla + tt * DK + c0) = float4{sa[0], sa[1], sa[2], sa[3]};
}

template <int DK, int DV, typename Tin, bool G2>
int launch_gbwd_t(const GatedBackwardArgs& a, hipStream_t s) {
  constexpr int RS = DV / kBwdSliceRows;
  const int BH = a.B * a.H;
  const GBufs wb = gbufs(a.ws, BH, a.T, DK, DV, G2);
  GParams p{BH, a.T, a.eta, a.scale, a.q, a.k, a.v, a.b, a.w, a.beta, a.r, a.log_alpha,
            a.d0, a.S0, a.dout, a.dST, wb, a.dv, a.dw, a.dS0};
  const int grid = bwd_grid(BH, RS);
  const int tk1 = ktimer_before(s, G2 ? "gdn2_bwd_record" : "gated_bwd_record");
  hipLaunchKernelGGL((gated_bwd_record_kernel<DK, DV, Tin, G2>), dim3(grid), dim3(kBwdThreads),
                     0, s, p);
  ktimer_after(s, tk1);
  int rc = (int)hipGetLastError();
  if (rc) return rc;
  const int tk2 = ktimer_before(s, G2 ? "gdn2_bwd" : "gated_bwd");
  hipLaunchKernelGGL((gated_bwd_kernel<DK, DV, Tin, G2>), dim3(grid), dim3(kBwdThreads), 0, s,
                     p);
  ktimer_after(s, tk2);
  rc = (int)hipGetLastError();
  if (rc) return rc;
  if constexpr (G2) {
    const size_t items = (size_t)BH * a.T * (DK / 4);
    if (items > 0) {
      const int tk3 = ktimer_before(s, "gdn2_bwd_out");
      hipLaunchKernelGGL((gdn2_bwd_out_kernel<DK, DV, Tin>), dim3((items + 255) / 256),
                         dim3(256), 0, s, BH, a.T, (const Tin*)a.k, (const Tin*)a.b, a.scale,
                         wb.sh, a.dq, a.dk, a.db, a.dla);
      ktimer_after(s, tk3);
    }
  } else {
    const int tk3 = ktimer_before(s, "gated_bwd_learner");
    LearnerArgs la{a.T, a.k, a.beta, a.r, a.eta, a.scale, a.ddT, wb.d, wb.sh,
                   a.dq, a.dk, a.dbeta, a.dr, a.deta, a.dd0, a.dla};
    hipLaunchKernelGGL((osdn_bwd_learner_kernel<DK, DV, Tin, true>), dim3(BH),
                       dim3(kLearnThreads), 0, s, la);
    ktimer_after(s, tk3);
  }
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
