// Chunkwise WY delta-rule engine: phase 2 of the OSDN forward and the Gated
// DeltaNet-2 forward.
//
// One engine serves every update of the form (state S: Dv x Dk; per chunk of
// C tokens with entry state S0)
//   A  = strictLower(diag(rs) Y X^T)          chunk Gram (read keys Y, write keys X)
//   T  = (I + A)^-1
//   W  = T diag(rs) (Z - Y S0^T)              row t of W is the token-t write
//   O  = Q S0^T + (Q X^T masked to i <= t) W  inclusive readout
//   S1 = S0 diag(g) + W^T X'                  exit state (g: exit decay)
//
// OSDN ([OSDN-it] 2.1): Y = K, X = X' = K~ (the preconditioned keys: K~
// replaces K in the Gram matrix and the intra-chunk scores), Z = V,
// rs = beta, g = 1; the rewrite of S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t)
// k~_t^T.
//
// GDN-2 ([GDN2-it] method, parts 1-3): S_t = (I - k_t e_t^T) Diag(alpha_t)
// S_{t-1} + k_t z_t^T with e = b*k, z = w*v, state Dk x Dv (handled here as
// its transpose). With gamma_t = prod_{j<=t} alpha_j inside the chunk the
// per-channel decay is absorbed into the factors, which leaves an undecayed
// delta rule with read key y_t = gamma_t*b_t*k_t, write key x_t = k_t/gamma_t,
// value z_t, query gamma_t*q_t, exit keys x'_t = k_t*gamma_C/gamma_t and exit
// decay g = gamma_C; rs = 1.
//
// Work decomposition: one workgroup (4 waves) per (batch, head, VT-wide value
// tile) walks the chunks in order; the VT x Dk state slice lives in fp32 MFMA
// accumulators. Value tiles are independent given the keys, so the
// V-independent chunk quantities (A, T, Q X^T) are recomputed per tile rather
// than written to and re-read from HBM. The next chunk's inputs are fetched
// into registers while the current chunk computes.
//
// T = (I + A)^-1: 16x16 diagonal blocks by fp32 forward substitution (one
// lane per column), then recursive doubling, merging pairs of s x s inverses
// into 2s x 2s ones with T21 = -T22 A21 T11 on MFMA.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace osdn {

struct OsdnVariant {};
struct Gdn2Variant {};

template <int DK, int C, int VT, typename Tin>
struct WyCfg {
  static constexpr int NW = 4, NT = 256;
  static constexpr int PAD = sizeof(Tin) == 2 ? 8 : 4;
  static constexpr int LDK = DK + PAD;
  static constexpr int LDC = C + PAD;
  static constexpr int LDR = VT + PAD;         // rows of R and W ([C][VT])
  static constexpr int LDS16 = 16 + PAD;       // doubling scratch ([C/2][16])
  static constexpr int TB = C / 16, VB = VT / 16, DB = DK / 16;
  static constexpr int VEC = 16 / sizeof(Tin);
  static constexpr int NCB = DK / VEC;         // 16-byte blocks per key row
  static constexpr size_t E = sizeof(Tin);
  static constexpr size_t oX = 0;
  static constexpr size_t oY = oX + (size_t)C * LDK * E;
  static constexpr size_t oQ = oY + (size_t)C * LDK * E;
  static constexpr size_t oS = oQ + (size_t)C * LDK * E;
  static constexpr size_t oZ = oS + (size_t)VT * LDK * E;
  static constexpr size_t oRS = oZ + (size_t)C * VT * E;
  static constexpr size_t oG = oRS + (size_t)C * 4;
  // fp32 diagonal 16x16 blocks of A, each stored transposed (column-major)
  static constexpr int LDD = 20;
  static constexpr size_t oA = oG + (size_t)DK * 4;
  static constexpr size_t oAb = oA + (size_t)TB * 16 * LDD * 4;
  static constexpr size_t oTb = oAb + (size_t)C * LDC * E;
  static constexpr size_t oYs = oTb + (size_t)C * LDC * E;
  static constexpr size_t oP = oYs + (size_t)NW * (C / 2) * LDS16 * E;
  static constexpr size_t oR = oP + (size_t)C * LDC * E;
  static constexpr size_t oW = oR + (size_t)C * LDR * E;
  static constexpr size_t bytes = oW + (size_t)C * LDR * E;
  static constexpr bool fits = bytes <= 163840;
  // State tiles per wave: every value tile times a contiguous run of DPW key
  // tiles.
  static constexpr int DPW = (DB + NW - 1) / NW;
  static constexpr int NS = VB * DPW;
  static constexpr int NLK = (C * DK / VEC + NT - 1) / NT;
  static constexpr int NLV = (C * VT / VEC + NT - 1) / NT;
  // GDN-2 decay pass: TPC threads per key channel, each over C/TPC tokens
  static constexpr int TPC = NT / DK;
  static constexpr int TPT = C / TPC;
};

struct SmemPtrs {
  void *X, *Y, *Q, *Z;
  float *rs, *g;
};

// ---------------------------------------------------------------------------
// Per-variant chunk inputs, fetched into registers one chunk ahead.
// ---------------------------------------------------------------------------
template <class V, int DK, int C, int VT, typename Tin>
struct ChunkRegs;

// OSDN: k, k~, q (row-major [C][Dk]), v, beta.
template <int DK, int C, int VT, typename Tin>
struct ChunkRegs<OsdnVariant, DK, C, VT, Tin> {
  using G = WyCfg<DK, C, VT, Tin>;
  uint4 k[G::NLK], kt[G::NLK], q[G::NLK], v[G::NLV];
  float beta;

  __device__ __forceinline__ void load(const ChunkArgs& p, int bh, size_t t0,
                                       int valid, int v0) {
    const Tin* kp = (const Tin*)p.k;
    const Tin* ktp = (const Tin*)p.ktilde;
    const Tin* qp = (const Tin*)p.q;
    const Tin* vp = (const Tin*)p.v;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < G::NLK; ++i) {
      const int e = tid + i * G::NT;
      const uint4 z = {0u, 0u, 0u, 0u};
      k[i] = z; kt[i] = z; q[i] = z;
      if (e < C * G::NCB) {
        const int rr = e / G::NCB, cc = (e % G::NCB) * G::VEC;
        if (rr < valid) {
          const size_t g = (t0 + rr) * DK + cc;
          k[i] = *reinterpret_cast<const uint4*>(kp + g);
          q[i] = *reinterpret_cast<const uint4*>(qp + g);
          kt[i] = *reinterpret_cast<const uint4*>(ktp + g);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < G::NLV; ++i) {
      const int e = tid + i * G::NT;
      const int rr = e / (VT / G::VEC), cc = (e % (VT / G::VEC)) * G::VEC;
      v[i] = uint4{0u, 0u, 0u, 0u};
      if (e < C * VT / G::VEC && rr < valid)
        v[i] = *reinterpret_cast<const uint4*>(vp + (t0 + rr) * p.Dv + v0 + cc);
    }
    beta = (tid < valid) ? p.beta[t0 + tid] : 0.f;
  }

  __device__ __forceinline__ void store(const SmemPtrs& s) const {
    Tin* Xs = (Tin*)s.X;
    Tin* Ys = (Tin*)s.Y;
    Tin* Qs = (Tin*)s.Q;
    Tin* Zs = (Tin*)s.Z;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < G::NLK; ++i) {
      const int e = tid + i * G::NT;
      if (e < C * G::NCB) {
        const int rr = e / G::NCB, cc = (e % G::NCB) * G::VEC;
        *reinterpret_cast<uint4*>(Ys + rr * G::LDK + cc) = k[i];
        *reinterpret_cast<uint4*>(Qs + rr * G::LDK + cc) = q[i];
        *reinterpret_cast<uint4*>(Xs + rr * G::LDK + cc) = kt[i];
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
    if (tid < C) s.rs[tid] = beta;
  }

  __device__ __forceinline__ void transform(const SmemPtrs&) const {}
};

// GDN-2: k, q, b staged raw (row-major) into the X, Q, Y buffers, z = w*v,
// and log alpha held by the threads of the decay pass (TPC threads per key
// channel, each over a contiguous run of TPT tokens).
template <int DK, int C, int VT, typename Tin>
struct ChunkRegs<Gdn2Variant, DK, C, VT, Tin> {
  using G = WyCfg<DK, C, VT, Tin>;
  uint4 k[G::NLK], q[G::NLK], b[G::NLK], v[G::NLV], w[G::NLV];
  float la[G::TPT];

  __device__ __forceinline__ static void chan(int& c, int& part) {
    // lanes l and l + 64/TPC (within one wave) share a channel
    constexpr int CPW = 64 / G::TPC;            // channels per wave
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    c = wave * CPW + lane % CPW;
    part = lane / CPW;
  }

  __device__ __forceinline__ void load(const ChunkArgs& p, int bh, size_t t0,
                                       int valid, int v0) {
    const Tin* kp = (const Tin*)p.k;
    const Tin* qp = (const Tin*)p.q;
    const Tin* bp = (const Tin*)p.b;
    const Tin* vp = (const Tin*)p.v;
    const Tin* wp = (const Tin*)p.w;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < G::NLK; ++i) {
      const int e = tid + i * G::NT;
      const uint4 z = {0u, 0u, 0u, 0u};
      k[i] = z; q[i] = z; b[i] = z;
      if (e < C * G::NCB) {
        const int rr = e / G::NCB, cc = (e % G::NCB) * G::VEC;
        if (rr < valid) {
          const size_t g = (t0 + rr) * DK + cc;
          k[i] = *reinterpret_cast<const uint4*>(kp + g);
          q[i] = *reinterpret_cast<const uint4*>(qp + g);
          b[i] = *reinterpret_cast<const uint4*>(bp + g);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < G::NLV; ++i) {
      const int e = tid + i * G::NT;
      const int rr = e / (VT / G::VEC), cc = (e % (VT / G::VEC)) * G::VEC;
      v[i] = uint4{0u, 0u, 0u, 0u};
      w[i] = v[i];
      if (e < C * VT / G::VEC && rr < valid) {
        const size_t g = (t0 + rr) * p.Dv + v0 + cc;
        v[i] = *reinterpret_cast<const uint4*>(vp + g);
        w[i] = *reinterpret_cast<const uint4*>(wp + g);
      }
    }
    int c, part;
    chan(c, part);
#pragma unroll
    for (int m = 0; m < G::TPT; ++m) {
      const int t = part * G::TPT + m;
      la[m] = (t < valid) ? p.log_alpha[(t0 + t) * DK + c] : 0.f;
    }
  }

  __device__ __forceinline__ void store(const SmemPtrs& s) const {
    Tin* Xs = (Tin*)s.X;
    Tin* Ys = (Tin*)s.Y;
    Tin* Qs = (Tin*)s.Q;
    Tin* Zs = (Tin*)s.Z;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < G::NLK; ++i) {
      const int e = tid + i * G::NT;
      if (e < C * G::NCB) {
        const int rr = e / G::NCB, cc = (e % G::NCB) * G::VEC;
        *reinterpret_cast<uint4*>(Xs + rr * G::LDK + cc) = k[i];
        *reinterpret_cast<uint4*>(Qs + rr * G::LDK + cc) = q[i];
        *reinterpret_cast<uint4*>(Ys + rr * G::LDK + cc) = b[i];
      }
    }
#pragma unroll
    for (int i = 0; i < G::NLV; ++i) {
      const int e = tid + i * G::NT;
      if (e < C * VT / G::VEC) {
        const int rr = e / (VT / G::VEC), cc = (e % (VT / G::VEC)) * G::VEC;
        const Tin* vv = reinterpret_cast<const Tin*>(&v[i]);
        const Tin* ww = reinterpret_cast<const Tin*>(&w[i]);
        Tin zz[G::VEC];
#pragma unroll
        for (int u = 0; u < G::VEC; ++u)
          zz[u] = from_f32<Tin>(to_f32(ww[u]) * to_f32(vv[u]));
        *reinterpret_cast<uint4*>(Zs + rr * VT + cc) =
            *reinterpret_cast<const uint4*>(zz);
      }
    }
    if (tid < C) s.rs[tid] = 1.f;
  }

  // Decay pass (after the raw operands are in LDS): cumulative log decay per
  // channel, then X = k/gamma, Y = gamma*b*k, Q = gamma*q in place, and the
  // exit decay g = gamma_C (the exit keys are X' = X diag(g)).
  __device__ __forceinline__ void transform(const SmemPtrs& s) const {
    Tin* Xs = (Tin*)s.X;
    Tin* Ys = (Tin*)s.Y;
    Tin* Qs = (Tin*)s.Q;
    constexpr int CPW = 64 / G::TPC;
    int c, part;
    chan(c, part);
    // prefix of log alpha: within this thread's run, then across the runs
    float lam[G::TPT];
    float run = 0.f;
#pragma unroll
    for (int m = 0; m < G::TPT; ++m) {
      run += la[m];
      lam[m] = run;
    }
    float incl = run;  // inclusive prefix over the runs of this channel
#pragma unroll
    for (int d = 1; d < G::TPC; d <<= 1) {
      const float y = __shfl_up(incl, d * CPW, 64);
      if (part >= d) incl += y;
    }
    const float excl = incl - run;
    const float total = __shfl(incl, (G::TPC - 1) * CPW + (threadIdx.x & 63) % CPW, 64);
    const float gC = __expf(total);
    // Batches of BT tokens: all loads of a batch are issued before its
    // arithmetic and stores; 1/gamma by the hardware reciprocal.
    constexpr int BT = G::TPT >= 8 ? 8 : G::TPT;
#pragma unroll
    for (int m0 = 0; m0 < G::TPT; m0 += BT) {
      const int tb0 = part * G::TPT + m0;
      float kk[BT], bb[BT], qq[BT];
#pragma unroll
      for (int u = 0; u < BT; ++u) {
        kk[u] = to_f32(Xs[(tb0 + u) * G::LDK + c]);
        bb[u] = to_f32(Ys[(tb0 + u) * G::LDK + c]);
        qq[u] = to_f32(Qs[(tb0 + u) * G::LDK + c]);
      }
#pragma unroll
      for (int u = 0; u < BT; ++u) {
        const float l = excl + lam[m0 + u];
        const float gam = __expf(l);
        const float igam = __builtin_amdgcn_rcpf(gam);
        Xs[(tb0 + u) * G::LDK + c] = from_f32<Tin>(kk[u] * igam);
        Ys[(tb0 + u) * G::LDK + c] = from_f32<Tin>(gam * bb[u] * kk[u]);
        Qs[(tb0 + u) * G::LDK + c] = from_f32<Tin>(gam * qq[u]);
      }
    }
    if (part == 0) s.g[c] = gC;
  }
};

// ---------------------------------------------------------------------------
// The engine
// ---------------------------------------------------------------------------
template <class V, int DK, int C, int VT, typename Tin>
__global__ __launch_bounds__(256) void wy_engine_kernel(ChunkArgs p) {
  using G = WyCfg<DK, C, VT, Tin>;
  constexpr bool kGdn2 = std::is_same<V, Gdn2Variant>::value;
  constexpr int LDK = G::LDK, LDC = G::LDC, LDR = G::LDR, LDS16 = G::LDS16;
  constexpr int TB = G::TB, VB = G::VB, DB = G::DB;
  __shared__ __attribute__((aligned(16))) unsigned char smem[G::bytes];
  Tin* Xs = reinterpret_cast<Tin*>(smem + G::oX);
  Tin* Ys = reinterpret_cast<Tin*>(smem + G::oY);
  Tin* Qs = reinterpret_cast<Tin*>(smem + G::oQ);
  Tin* Ss = reinterpret_cast<Tin*>(smem + G::oS);
  Tin* Zs = reinterpret_cast<Tin*>(smem + G::oZ);
  float* rs = reinterpret_cast<float*>(smem + G::oRS);
  float* gC = reinterpret_cast<float*>(smem + G::oG);
  float* Am = reinterpret_cast<float*>(smem + G::oA);
  Tin* Ab = reinterpret_cast<Tin*>(smem + G::oAb);
  Tin* Tb = reinterpret_cast<Tin*>(smem + G::oTb);
  Tin* Ysc = reinterpret_cast<Tin*>(smem + G::oYs);
  Tin* Pb = reinterpret_cast<Tin*>(smem + G::oP);
  Tin* Rm = reinterpret_cast<Tin*>(smem + G::oR);
  Tin* Wm = reinterpret_cast<Tin*>(smem + G::oW);
  const SmemPtrs sp{Xs, Ys, Qs, Zs, rs, gC};

  const int T = p.T, Dv = p.Dv;
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
  Tin* o = (Tin*)p.o;

  // Blocks above the diagonal of T and P stay zero.
  for (int e = tid; e < C * C; e += G::NT) {
    const int rr = e / C, cc = e % C;
    if ((cc >> 4) > (rr >> 4)) {
      Tb[rr * LDC + cc] = zero;
      Pb[rr * LDC + cc] = zero;
    }
  }

  // Persistent state slice S[v][dk] (v in this tile), fp32, MFMA layout.
  // OSDN stores the state [Dv][Dk]; GDN-2 stores it [Dk][Dv].
  auto sidx = [&](int vv, int kk) -> size_t {
    return kGdn2 ? ((size_t)bh * DK + kk) * Dv + v0 + vv
                 : ((size_t)bh * Dv + v0 + vv) * DK + kk;
  };
  f32x4 Sacc[G::NS];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb) {
#pragma unroll
    for (int u = 0; u < G::DPW; ++u) {
      const int db = wave * G::DPW + u;
      f32x4& acc = Sacc[vb * G::DPW + u];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = 0.f;
        if (db < DB && p.S0)
          x = p.S0[sidx(vb * 16 + acc_row(i), db * 16 + acc_col())];
        acc[i] = x;
      }
      if (db < DB) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Ss[(vb * 16 + acc_row(i)) * LDK + db * 16 + acc_col()] =
              from_f32<Tin>(acc[i]);
      }
    }
  }

  const int nchunks = (T + C - 1) / C;
  ChunkRegs<V, DK, C, VT, Tin> regs;
  if (nchunks > 0) regs.load(p, bh, row0, min(C, T), v0);

  for (int j = 0; j < nchunks; ++j) {
    const size_t t0 = row0 + (size_t)j * C;
    const int valid = min(C, T - j * C);
    // ---- S1: operands of chunk j into LDS; prefetch chunk j+1 -------------
    regs.store(sp);
    if constexpr (kGdn2) {
      __syncthreads();
      regs.transform(sp);
    }
    if (j + 1 < nchunks)
      regs.load(p, bh, t0 + C, min(C, T - (j + 1) * C), v0);
    __syncthreads();

    // ---- S2: Gram A, scores P, RHS = rs (Z - Y S0^T), Q S0^T; diagonal
    // blocks of T. Wave w owns the 16-row block w: its read-key and query
    // fragments stay in registers across all tiles of the row.
    f32x4 Oacc[VB];
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) Oacc[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (wave < TB) {
      const int rb = wave;
      Frag<DK, Tin> fy, fq;
      fy.load(Ys + rb * 16 * LDK, LDK);
      fq.load(Qs + rb * 16 * LDK, LDK);
      float rsr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) rsr[i] = rs[rb * 16 + acc_row(i)];
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        if (b <= rb) {
          Frag<DK, Tin> fx;
          fx.load(Xs + b * 16 * LDK, LDK);
          f32x4 aa = {0.f, 0.f, 0.f, 0.f}, pa = {0.f, 0.f, 0.f, 0.f};
          mma(aa, fy, fx);
          mma(pa, fq, fx);
          if (b < rb) {
            // off-diagonal tile: operand copy for the doubling merges
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int rr = rb * 16 + acc_row(i), cc = b * 16 + acc_col();
              Ab[rr * LDC + cc] = from_f32<Tin>(rsr[i] * aa[i]);
              Pb[rr * LDC + cc] = from_f32<Tin>(pa[i]);
            }
          } else {
            // diagonal tile: fp32, transposed, strictly lower part only
            float4 col;
            col.x = acc_row(0) > acc_col() ? rsr[0] * aa[0] : 0.f;
            col.y = acc_row(1) > acc_col() ? rsr[1] * aa[1] : 0.f;
            col.z = acc_row(2) > acc_col() ? rsr[2] * aa[2] : 0.f;
            col.w = acc_row(3) > acc_col() ? rsr[3] * aa[3] : 0.f;
            *reinterpret_cast<float4*>(Am + (rb * 16 + acc_col()) * G::LDD +
                                       acc_row(0)) = col;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int rr = rb * 16 + acc_row(i), cc = b * 16 + acc_col();
              Pb[rr * LDC + cc] = from_f32<Tin>(cc <= rr ? pa[i] : 0.f);
            }
          }
        }
      }
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        Frag<DK, Tin> fs;
        fs.load(Ss + vb * 16 * LDK, LDK);
        f32x4 ka = {0.f, 0.f, 0.f, 0.f};
        mma(ka, fy, fs);
        mma(Oacc[vb], fq, fs);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = rb * 16 + acc_row(i), cc = vb * 16 + acc_col();
          Rm[rr * LDR + cc] =
              from_f32<Tin>(rsr[i] * (to_f32(Zs[rr * VT + cc]) - ka[i]));
        }
      }
      // Diagonal block rb of T = (I + A)^-1 by fp32 forward substitution:
      // lane c < 16 owns column c; pending sums are updated as soon as each
      // entry is final, so the dependent chain is 15 FMAs long. Column m of
      // the block is read as four broadcast 16-byte loads. The block was
      // written by this wave, so only a wave-level LDS ordering is needed.
      wave_lds_sync();
      if (lane < 16) {
        const int c = lane;
        const float* Acol = Am + rb * 16 * G::LDD;
        float x[16], sv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[i] = (i == c) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          x[m] = sv[m];
          float col[16];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const float4 v4 = *reinterpret_cast<const float4*>(Acol + m * G::LDD + 4 * q4);
            col[4 * q4] = v4.x; col[4 * q4 + 1] = v4.y;
            col[4 * q4 + 2] = v4.z; col[4 * q4 + 3] = v4.w;
          }
#pragma unroll
          for (int i = m + 1; i < 16; ++i) sv[i] -= col[i] * x[m];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
          Tb[(rb * 16 + i) * LDC + rb * 16 + c] = from_f32<Tin>(x[i]);
      }
    }
    __syncthreads();

    // ---- S4: recursive doubling, T21 = -T22 (A21 T11) ----------------------
    // One job = one 16-wide column of T21 in one pair: the wave computes that
    // column of Y = A21 T11 (into its own scratch, row-major) and then the
    // same column of T21 = -T22 Y, so the two stages need no barrier between
    // them. The right operands (T11, Y) are read k-major.
    {
      Tin* ys = Ysc + wave * (C / 2) * LDS16;
#pragma unroll
      for (int s = 16; s < C; s *= 2) {
        const int nt = s / 16;
        const int jobs = (C / (2 * s)) * nt;
        for (int job = wave; job < jobs; job += G::NW) {
          const int pp = job / nt, c = job % nt;
          const int rb = 2 * s * pp + s, cb = 2 * s * pp;
          for (int r = 0; r < nt; ++r) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int kk = 0; kk < s; kk += 16) {
              Frag<16, Tin> fa, fb;
              fa.load(Ab + (rb + r * 16) * LDC + cb + kk, LDC);
              fb.load_kmajor(Tb + (cb + kk) * LDC + cb + c * 16, LDC);
              mma(acc, fa, fb);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
              ys[(r * 16 + acc_row(i)) * LDS16 + acc_col()] = from_f32<Tin>(acc[i]);
          }
          wave_lds_sync();
          for (int r = 0; r < nt; ++r) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int kk = 0; kk < s; kk += 16) {
              Frag<16, Tin> fa, fb;
              fa.load(Tb + (rb + r * 16) * LDC + rb + kk, LDC);
              fb.load_kmajor(ys + kk * LDS16, LDS16);
              mma(acc, fa, fb);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
              Tb[(rb + r * 16 + acc_row(i)) * LDC + cb + c * 16 + acc_col()] =
                  from_f32<Tin>(-acc[i]);
          }
          // the scratch is rewritten by this wave's next job
          wave_lds_sync();
        }
        __syncthreads();
      }
    }

    // ---- S5: W = T RHS (row-major [C][VT]) --------------------------------
    for (int job = wave; job < TB * VB; job += G::NW) {
      const int tb = job / VB, vb = job % VB;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      Frag<C, Tin> ft, fr;
      ft.load(Tb + tb * 16 * LDC, LDC);
      fr.load_kmajor(Rm + vb * 16, LDR);
      mma(acc, ft, fr);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Wm[(tb * 16 + acc_row(i)) * LDR + vb * 16 + acc_col()] = from_f32<Tin>(acc[i]);
    }
    __syncthreads();

    // ---- S6: O += P W (store), S = S diag(g) + W^T X' -----------------------
    if (wave < TB) {
      const int tb = wave;
      Frag<C, Tin> fp;
      fp.load(Pb + tb * 16 * LDC, LDC);
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        Frag<C, Tin> fw;
        fw.load_kmajor(Wm + vb * 16, LDR);
        mma(Oacc[vb], fp, fw);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = tb * 16 + acc_row(i);
          if (rr < valid)
            o[(t0 + rr) * Dv + v0 + vb * 16 + acc_col()] =
                from_f32<Tin>(p.scale * Oacc[vb][i]);
        }
      }
    }
    // State tiles (vb, db): wave w takes a contiguous run of db for every vb,
    // so each W^T and X fragment is loaded once per wave; both are read
    // k-major (token rows) from their row-major tiles. GDN-2 applies the exit
    // decay after the product: g (S + W^T X) = S diag(g) + W^T X'.
    {
      constexpr int DPW = G::DPW;
      Frag<C, Tin> fw[VB];
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) fw[vb].load_kmajor(Wm + vb * 16, LDR);
#pragma unroll
      for (int u = 0; u < DPW; ++u) {
        const int db = wave * DPW + u;
        if (db < DB) {
          Frag<C, Tin> fx;
          fx.load_kmajor(Xs + db * 16, LDK);
#pragma unroll
          for (int vb = 0; vb < VB; ++vb) {
            f32x4& acc = Sacc[vb * G::DPW + u];
            mma(acc, fw[vb], fx);
            if constexpr (kGdn2) {
              const float gd = gC[db * 16 + acc_col()];
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[i] *= gd;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
              Ss[(vb * 16 + acc_row(i)) * LDK + db * 16 + acc_col()] =
                  from_f32<Tin>(acc[i]);
          }
        }
      }
    }
    __syncthreads();
  }

  if (p.ST) {
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
#pragma unroll
      for (int u = 0; u < G::DPW; ++u) {
        const int db = wave * G::DPW + u;
        if (db < DB) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            p.ST[sidx(vb * 16 + acc_row(i), db * 16 + acc_col())] =
                Sacc[vb * G::DPW + u][i];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------
template <class V, int DK, int C, int VT, typename Tin>
static int launch_cfg(const ChunkArgs& a, hipStream_t s) {
  if constexpr (!WyCfg<DK, C, VT, Tin>::fits) {
    return -1;
  } else {
    const int BH = a.B * a.H;
    dim3 grid(BH * (a.Dv / VT)), block(256);
    hipLaunchKernelGGL((wy_engine_kernel<V, DK, C, VT, Tin>), grid, block, 0, s,
                       a);
    return (int)hipGetLastError();
  }
}

// Value-tile width: 32 columns when that already gives one workgroup per
// compute unit (256 CUs), else 16 for more parallelism.
static int pick_vt(int BH, int Dv) { return (BH * (Dv / 32) >= 256) ? 32 : 16; }

template <class V, int DK, int C, typename Tin>
static int launch_c(const ChunkArgs& a, hipStream_t s) {
  if (pick_vt(a.B * a.H, a.Dv) == 32) return launch_cfg<V, DK, C, 32, Tin>(a, s);
  return launch_cfg<V, DK, C, 16, Tin>(a, s);
}

template <class V, int DK, typename Tin>
static int launch_dk(const ChunkArgs& a, hipStream_t s) {
  switch (a.chunk) {
    case 16: return launch_c<V, DK, 16, Tin>(a, s);
    case 32: return launch_c<V, DK, 32, Tin>(a, s);
    case 64: return launch_c<V, DK, 64, Tin>(a, s);
  }
  return -1;
}

template <class V>
static int launch_variant(const ChunkArgs& a, hipStream_t s) {
  if (a.bf16) {
    switch (a.Dk) {
      case 32: return launch_dk<V, 32, __bf16>(a, s);
      case 64: return launch_dk<V, 64, __bf16>(a, s);
      case 128: return launch_dk<V, 128, __bf16>(a, s);
    }
  } else {
    switch (a.Dk) {
      case 32: return launch_dk<V, 32, float>(a, s);
      case 64: return launch_dk<V, 64, float>(a, s);
      case 128: return launch_dk<V, 128, float>(a, s);
    }
  }
  return -1;
}

int launch_osdn_chunk(const ChunkArgs& a, hipStream_t s) {
  return launch_variant<OsdnVariant>(a, s);
}

int launch_gdn2_chunk(const ChunkArgs& a, hipStream_t s) {
  return launch_variant<Gdn2Variant>(a, s);
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

// The GDN-2 decay pass splits each chunk's tokens over 256/Dk threads per
// channel, so the chunk must hold at least that many tokens.
bool gdn2_chunk_supported(int Dk, int chunk, int bf16) {
  return osdn_chunk_supported(Dk, chunk, bf16) && chunk >= 256 / Dk;
}

}  // namespace osdn
