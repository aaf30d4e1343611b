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
// Split by dependence on S0. With P = Q X^T masked to i <= t,
//   Wk = T diag(rs) Y,  U = T diag(rs) Z,
// the chunk step is
//   W = U - Wk S0^T,    O = Q S0^T + P W,   S1 = S0 diag(g) + W^T X'.
// * prep: persistent workgroups of 8 waves over all chunks at once (the next
//   chunk is fetched while the current one computes) form Wk, U, P and X'
//   (GDN-2 also its decayed queries and exit decays) and write them to the
//   workspace in MFMA operand order.
//   T comes from 16x16 diagonal blocks by fp32 forward substitution (one lane
//   per column) and recursive doubling, T21 = -T22 A21 T11, on MFMA.
// * scan: one workgroup (4 waves) per (batch, head, VT-wide value tile) walks
//   the chunks in order with the VT x Dk state slice in fp32 MFMA
//   accumulators: W and Q S0^T from the state, then P W and the state update
//   from W, two barriers per chunk; each chunk's operands are fetched into
//   registers during the step before (two register sets used in turn).
#include <algorithm>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace osdn {

struct OsdnVariant {};
struct Gdn2Variant {};
// OSDN with the preconditioned keys formed in the engine from the raw keys,
// the phase-1 chunk records (gate prefix, step sizes) and the entry values
// of d: K~_t = d_t * k_t, with d_t from the preconditioner's own recursion
// inside the chunk, d_{t+1} = r_t d_t + g_t (k_t * k_t), in fp32 from the
// entry value ([OSDN-it] 2.2-2.3). Requires chunk == the phase-1 chunk.
struct OsdnFusedVariant {};
// OSDN on a backbone with per-key-channel decay (Kimi-style; a Gated
// DeltaNet scalar decay is the case of equal channels): S_t = S_{t-1}
// Diag(alpha_t) + beta_t (v_t - S_{t-1} Diag(alpha_t) k_t) k~_t^T. The decay
// is absorbed as for GDN-2, with read key y_t = gamma_t*beta_t*k_t, write key
// x_t = k~_t/gamma_t, value beta_t v_t, query gamma_t*q_t, exit keys
// k~_t*gamma_C/gamma_t and exit decay gamma_C; the state is stored [Dv, Dk].
struct OsdnGatedVariant {};
// The same with the preconditioned keys formed in the engine, as for
// OsdnFusedVariant (chunk == the phase-1 chunk); K~ is formed first, then
// the decay pass turns it into K~/gamma.
struct OsdnGatedFusedVariant {};

// Variants whose chunk operands carry a per-channel decay.
template <class V>
constexpr bool kDecayVariant = std::is_same<V, Gdn2Variant>::value ||
                               std::is_same<V, OsdnGatedVariant>::value ||
                               std::is_same<V, OsdnGatedFusedVariant>::value;
// Variants that form K~ from the raw keys and the phase-1 records.
template <class V>
constexpr bool kFusedVariant = std::is_same<V, OsdnFusedVariant>::value ||
                               std::is_same<V, OsdnGatedFusedVariant>::value;

// Four consecutive elements of the storage dtype as one LDS access.
template <typename Tin>
struct alignas(4 * sizeof(Tin)) RawQuad {
  Tin v[4];
};

// Two consecutive key channels of one token as one LDS access, unpacked to
// fp32 and packed back (bf16: round to nearest even).
template <typename Tin>
struct KeyPairOf;
template <>
struct KeyPairOf<__bf16> {
  using T = unsigned;
  __device__ static float lo(T p) { return __uint_as_float(p << 16); }
  __device__ static float hi(T p) { return __uint_as_float(p & 0xffff0000u); }
  __device__ static T pack(float a, float b) {
    const __bf16 x = (__bf16)a, y = (__bf16)b;
    return (unsigned)__builtin_bit_cast(unsigned short, x) |
           ((unsigned)__builtin_bit_cast(unsigned short, y) << 16);
  }
};
template <>
struct KeyPairOf<float> {
  using T = float2;
  __device__ static float lo(T p) { return p.x; }
  __device__ static float hi(T p) { return p.y; }
  __device__ static T pack(float a, float b) { return float2{a, b}; }
};

// Per-chunk operands in the workspace, each [B*H*nchunks][...] in the
// storage dtype: Wk as 16-row A fragments (row block tb at tb*16*Dk); the
// scores P as 16-row A fragments (row block tb at tb*16*C) and X' as k-major
// B fragments (channel block db at db*16*C), both over the tokens in the
// permuted order of Frag::load_perm, which P's accumulator tiles give
// directly; U as accumulator tiles, adjacent value tiles interleaved in
// pairs (u_tile). GDN-2
// adds the decayed queries Q^ (like Wk) and the exit decays g (fp32, Dk per
// chunk); OSDN's scan reads the queries themselves.
template <typename Tin>
struct WyBufs {
  Tin *wk, *xp, *u, *pp, *qh;
  float* g;
};

template <typename Tin>
static WyBufs<Tin> wy_bufs(void* ws, int BH, int nchunks, int C, int Dk, int Dv,
                           bool gdn2) {
  const size_t n = (size_t)BH * nchunks * C;
  Tin* b = static_cast<Tin*>(ws);
  WyBufs<Tin> w;
  w.wk = b;
  w.xp = w.wk + n * Dk;
  w.u = w.xp + n * Dk;
  w.pp = w.u + n * Dv;
  w.qh = gdn2 ? w.pp + n * C : nullptr;
  w.g = gdn2 ? reinterpret_cast<float*>(w.qh + n * Dk) : nullptr;
  return w;
}

size_t wy_workspace_bytes(int B, int H, int T, int Dk, int Dv, int chunk,
                          int bf16, int gdn2) {
  const size_t n = (size_t)B * H * ((T + chunk - 1) / chunk);
  const size_t e = bf16 ? 2 : 4;
  const size_t per = n * chunk * (2 * (size_t)Dk + (size_t)Dv + (size_t)chunk) * e;
  return gdn2 ? per + n * chunk * (size_t)Dk * e + n * Dk * 4 : per;
}

// Accumulator tile in the storage dtype, as fetched (converted at use, so
// that a prefetch is not waited on when it is issued).
template <typename Tin>
struct RawTile;
// U tiles are stored in pairs of adjacent value tiles, interleaved per lane:
// lane l's four values of tile (tb, ct) at u_tile(tb, ct) + 8 l, so that a
// wave fetches both tiles of a pair with one 16-byte access per lane (bf16).
__device__ __forceinline__ size_t u_tile(int tb, int ct, int VBT) {
  return (size_t)(tb * (VBT / 2) + (ct >> 1)) * 512 + (ct & 1) * 4;
}
template <>
struct RawTile<__bf16> {
  bf16x4 v;
  __device__ __forceinline__ void load(const __bf16* tile) {
    v = *reinterpret_cast<const bf16x4*>(tile + (threadIdx.x & 63) * 8);
  }
  __device__ __forceinline__ static void load_pair(const __bf16* tile, RawTile& a,
                                                   RawTile& b) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(tile + (threadIdx.x & 63) * 8);
    a.v = __builtin_shufflevector(x, x, 0, 1, 2, 3);
    b.v = __builtin_shufflevector(x, x, 4, 5, 6, 7);
  }
  __device__ __forceinline__ static void store(const f32x4& a, __bf16* tile) {
    bf16x4 h;
    h[0] = (__bf16)a[0]; h[1] = (__bf16)a[1]; h[2] = (__bf16)a[2]; h[3] = (__bf16)a[3];
    *reinterpret_cast<bf16x4*>(tile + (threadIdx.x & 63) * 8) = h;
  }
  __device__ __forceinline__ float operator[](int i) const { return (float)v[i]; }
};
template <>
struct RawTile<float> {
  f32x4 v;
  __device__ __forceinline__ void load(const float* tile) {
    v = *reinterpret_cast<const f32x4*>(tile + (threadIdx.x & 63) * 8);
  }
  __device__ __forceinline__ static void load_pair(const float* tile, RawTile& a,
                                                   RawTile& b) {
    a.load(tile);
    b.load(tile + 4);
  }
  __device__ __forceinline__ static void store(const f32x4& a, float* tile) {
    *reinterpret_cast<f32x4*>(tile + (threadIdx.x & 63) * 8) = a;
  }
  __device__ __forceinline__ float operator[](int i) const { return v[i]; }
};

// Scale the elements of an operand fragment in registers by a factor that
// depends on the element's position along the fragment's K dimension:
// row fragments (Frag::load: K = key channel) and k-major fragments in the
// permuted order (Frag::load_kmajor_perm: K = token) or the plain order
// (Frag::load_kmajor: K = token). f(k) gives the factor of index k.
template <int KEXT, typename F>
__device__ __forceinline__ void scale_row_frag(Frag<KEXT, __bf16>& fr, F f) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int i = 0; i < Frag<KEXT, __bf16>::N32; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) fr.v[i][e] = (__bf16)((float)fr.v[i][e] * f(32 * i + 8 * g + e));
  if constexpr (Frag<KEXT, __bf16>::R16) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      fr.t[e] = (__bf16)((float)fr.t[e] * f(32 * Frag<KEXT, __bf16>::N32 + 4 * g + e));
  }
}
template <int KEXT, typename F>
__device__ __forceinline__ void scale_row_frag(Frag<KEXT, float>& fr, F f) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int i = 0; i < KEXT / 4; ++i) fr.v[i] *= f(4 * i + g);
}
template <int KEXT, typename F>
__device__ __forceinline__ void scale_kperm_frag(Frag<KEXT, __bf16>& fr, F f) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int i = 0; i < Frag<KEXT, __bf16>::N32; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      fr.v[i][e] = (__bf16)((float)fr.v[i][e] *
                            f(32 * i + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4)));
  if constexpr (Frag<KEXT, __bf16>::R16) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      fr.t[e] = (__bf16)((float)fr.t[e] * f(32 * Frag<KEXT, __bf16>::N32 + 4 * g + e));
  }
}
template <int KEXT, typename F>
__device__ __forceinline__ void scale_kperm_frag(Frag<KEXT, float>& fr, F f) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int b = 0; b < KEXT / 16; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) fr.v[4 * b + i] *= f(16 * b + 4 * g + i);
}

// Maximum over the 64 lanes of a wave; every lane receives it.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

// Decay inside a chunk (variants whose operands carry a decay): with
// lambda_t the inclusive prefix of log alpha over the chunk, every factor
// exp(lambda_t - lambda_i), i <= t, is split at 16-token block boundaries so
// that each stored factor is at most 1: read keys and queries relative to the
// first token s_a of their block, write keys relative to the last token e_b
// of theirs, and tile (a, b) of the Gram matrix and of the scores takes the
// per-channel factor exp(lambda_{s_a} - lambda_{e_b}) on the write keys. That
// factor is at most 1 off the diagonal; on a diagonal tile it is the inverse
// decay over the block's 15 steps, which is used as is while its exponent
// stays below kExactDiag, else the tile is summed exactly, element by
// element, from the raw operands.
constexpr float kExactDiag = 60.f;

// ---------------------------------------------------------------------------
// prep
// ---------------------------------------------------------------------------
template <class V, int DK, int DV, int C, typename Tin>
struct PrepCfg {
  static constexpr bool kGdn2 = std::is_same<V, Gdn2Variant>::value;
  static constexpr bool kFused = kFusedVariant<V>;
  static constexpr int NW = 8, NT = 512;
  static constexpr int PAD = sizeof(Tin) == 2 ? 8 : 4;
  static constexpr int LDK = DK + PAD, LDV = DV + PAD, LDC = C + PAD;
  static constexpr int LDS16 = 16 + PAD;      // doubling scratch ([C/2][16])
  static constexpr int LDD = 20;              // fp32 diagonal blocks, transposed
  static constexpr int TB = C / 16, DB = DK / 16, VBT = DV / 16;
  static constexpr int VEC = 16 / sizeof(Tin);
  static constexpr size_t E = sizeof(Tin);
  static constexpr size_t oY = 0;
  static constexpr size_t oX = oY + (size_t)C * LDK * E;
  static constexpr size_t oQ = oX + (size_t)C * LDK * E;
  static constexpr size_t oZ = oQ + (size_t)C * LDK * E;
  static constexpr size_t oAb = oZ + (size_t)C * LDV * E;
  static constexpr size_t oTb = oAb + (size_t)C * LDC * E;
  static constexpr size_t oA = oTb + (size_t)C * LDC * E;
  static constexpr size_t oYs = oA + (size_t)TB * 16 * LDD * 4;
  static constexpr size_t oG = oYs + (size_t)NW * (C / 2) * LDS16 * E;
  // fused OSDN only: K~ comes from the preconditioner's recursion over NSEG
  // segments of the chunk (one lane per segment and key channel pair): the
  // segments' end values [NSEG][DK], step sizes g_t, entry d, gate factors
  // r_t = P_{t+1} / P_t and P_t / P_s (s the first token of t's segment)
  static constexpr int NSEG = kFused ? NW * (128 / DK) : 1;
  static constexpr int SEGL = C / NSEG > 0 ? C / NSEG : 1;
  static constexpr size_t oFe = oG + (size_t)DK * 4;
  static constexpr size_t oGs = oFe + (kFused ? (size_t)NSEG * DK * 4 : 0);
  static constexpr size_t oDs = oGs + (kFused ? (size_t)C * 4 : 0);
  static constexpr size_t oRt = oDs + (kFused ? (size_t)DK * 4 : 0);
  static constexpr size_t oRa = oRt + (kFused ? (size_t)C * 4 : 0);
  static constexpr size_t oEnd = oRa + (kFused ? (size_t)C * 4 : 0);
  static_assert(!kFused || C != kPrecondChunk || (128 % DK == 0 && C % NSEG == 0),
                "whole segments, one lane per segment and channel pair");
  // GDN-2 only: log alpha staged as fp32 rows, in a region of its own when
  // that fits, else over the Gram/inverse buffers (not in use yet during the
  // decay pass), whose zero blocks above the diagonal are then restored
  static constexpr int LDA = DK + 4;
  static constexpr size_t kLaBytes = kDecayVariant<V> ? (size_t)C * LDA * 4 : 0;
  static constexpr bool kLaOwn = oEnd + kLaBytes <= 163840;
  static constexpr bool kLaInGram = !kLaOwn && oAb + kLaBytes <= oG;
  static constexpr size_t oLa = kLaOwn ? oEnd : oAb;
  static constexpr size_t bytes = kLaOwn ? oEnd + kLaBytes : oEnd;
  // (the fused decay variant keeps its log alpha in a region of its own)
  static constexpr bool fits =
      bytes <= 163840 && (kLaOwn || (kLaInGram && !(kFused && kDecayVariant<V>)));
  // GDN-2 decay pass: TPC threads per key channel, each over TPT tokens
  static constexpr int TPC = NT / DK;
  static constexpr int TPT = C / TPC > 0 ? C / TPC : 1;
  // decay variants: per 16-token block, lambda at its first and last token
  // (fp32, [TB][DK] each), kept in the doubling scratch, which is dead from
  // the decay pass until the doubling starts
  static_assert(!kDecayVariant<V> ||
                    (size_t)NW * (C / 2) * LDS16 * E >= (size_t)2 * TB * DK * 4,
                "block decay table fits in the doubling scratch");
  static_assert(!kDecayVariant<V> || kLaOwn || oLa + kLaBytes <= oYs,
                "log alpha staged over the Gram buffers stays clear of the table");
};

// Raw operands of one chunk, fetched into registers while the previous chunk
// computes (padding rows are zero).
template <class V, int DK, int DV, int C, typename Tin>
struct PrepRegs {
  using G = PrepCfg<V, DK, DV, C, Tin>;
  static constexpr bool kGdn2 = std::is_same<V, Gdn2Variant>::value;
  static constexpr bool kFused = kFusedVariant<V>;
  static constexpr int VEC = G::VEC;
  static constexpr int NKB = C * (DK / VEC), NVB = C * (DV / VEC);
  static constexpr int NLK = (NKB + G::NT - 1) / G::NT;
  static constexpr int NLV = (NVB + G::NT - 1) / G::NT;
  uint4 k[NLK], q[NLK], x[kFused ? 1 : NLK], v[NLV], w[kGdn2 ? NLV : 1];
  float bk[NLK], bv[NLV];          // OSDN: beta of the row
  static constexpr int NLA = (C * DK / 4 + G::NT - 1) / G::NT;
  static constexpr bool kDecay = kDecayVariant<V>;
  uint4 la4[kDecay ? NLA : 1];     // decay variants: log alpha, 4 channels per load
  float plp, plp1, plps, pg, pd;   // fused OSDN: record entries, entry d
  int vrows;                       // valid rows of the fetched chunk

  // Loads are unconditional (rows past the sequence end read the last valid
  // row and are zeroed when staged), so that the compiler can count them and
  // the fetch is only waited on where the staging uses it.
  __device__ __forceinline__ void load(const ChunkArgs& p, int n, int nchunks) {
    load_a(p, n, nchunks);
    load_b(p, n, nchunks);
    load_c(p, n, nchunks);
  }
  // keys, queries (and the write or erase keys) with their beta
  __device__ __forceinline__ void load_a(const ChunkArgs& p, int n, int nchunks) {
    const int bh = n / nchunks, j = n - bh * nchunks;
    const int T = p.T, tid = threadIdx.x;
    const int valid = min(C, T - j * C);
    vrows = valid;
    const size_t t0 = (size_t)bh * T + (size_t)j * C;
    const Tin* xs = kGdn2 ? (const Tin*)p.b : (const Tin*)p.ktilde;
#pragma unroll
    for (int i = 0; i < NLK; ++i) {
      const int e = min(tid + i * G::NT, NKB - 1);
      const int rr = min(e / (DK / VEC), valid - 1), cc = (e % (DK / VEC)) * VEC;
      const size_t gi = (t0 + rr) * DK + cc;
      k[i] = *reinterpret_cast<const uint4*>((const Tin*)p.k + gi);
      q[i] = *reinterpret_cast<const uint4*>((const Tin*)p.q + gi);
      if constexpr (!kFused) x[i] = *reinterpret_cast<const uint4*>(xs + gi);
      if constexpr (!kGdn2) bk[i] = p.beta[t0 + rr];
    }
  }
  // the record entries (fused), values (and write gates) with their beta
  __device__ __forceinline__ void load_b(const ChunkArgs& p, int n, int nchunks) {
    const int bh = n / nchunks, j = n - bh * nchunks;
    const int T = p.T, Dv = p.Dv, tid = threadIdx.x;
    const int valid = min(C, T - j * C);
    const size_t t0 = (size_t)bh * T + (size_t)j * C;
    if constexpr (kFused) {
      // the phase-1 chunk of this engine chunk has the same index
      const float* rc = p.prec + (size_t)n * kRecStride;
      const int tt = min(tid, C - 1);
      plp = rc[kRecLp + tt];
      plp1 = rc[kRecLp + tt + 1];
      plps = rc[kRecLp + (tt / G::SEGL) * G::SEGL];
      pg = rc[kRecG + tt];
      pd = p.pdent[(size_t)n * DK + min(tid, DK - 1)];
    }
#pragma unroll
    for (int i = 0; i < NLV; ++i) {
      const int e = min(tid + i * G::NT, NVB - 1);
      const int rr = min(e / (DV / VEC), valid - 1), cc = (e % (DV / VEC)) * VEC;
      const size_t gi = (t0 + rr) * Dv + cc;
      v[i] = *reinterpret_cast<const uint4*>((const Tin*)p.v + gi);
      if constexpr (kGdn2)
        w[i] = *reinterpret_cast<const uint4*>((const Tin*)p.w + gi);
      else
        bv[i] = p.beta[t0 + rr];
    }
  }
  // the decays (decay variants)
  __device__ __forceinline__ void load_c(const ChunkArgs& p, int n, int nchunks) {
    const int bh = n / nchunks, j = n - bh * nchunks;
    const int T = p.T, tid = threadIdx.x;
    const int valid = min(C, T - j * C);
    const size_t t0 = (size_t)bh * T + (size_t)j * C;
    if constexpr (kDecay) {
#pragma unroll
      for (int i = 0; i < NLA; ++i) {
        const int e = min(tid + i * G::NT, C * DK / 4 - 1);
        const int rr = min(e / (DK / 4), valid - 1), cc = (e % (DK / 4)) * 4;
        la4[i] = *reinterpret_cast<const uint4*>(p.log_alpha + (t0 + rr) * DK + cc);
      }
    }
  }

  // OSDN: Y = beta*k, X = k~, Q = q, Z = beta*v. GDN-2: raw k, b, q and
  // Z = w*v (the decay pass forms X, Y and Q in place). Fused OSDN: X = raw
  // k (turned into K~ in place) and the record entries.
  __device__ __forceinline__ void store(Tin* Ys, Tin* Xs, Tin* Qs, Tin* Zs,
                                        unsigned char* smem) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NLK; ++i) {
      const int e = tid + i * G::NT;
      if (e < NKB) {
        const int rr = e / (DK / VEC), cc = (e % (DK / VEC)) * VEC;
        const bool live = rr < vrows;
        const uint4 kk = keep_or_zero(k[i], live);
        *reinterpret_cast<uint4*>(Qs + rr * G::LDK + cc) = keep_or_zero(q[i], live);
        if constexpr (kGdn2) {
          *reinterpret_cast<uint4*>(Xs + rr * G::LDK + cc) = kk;
          *reinterpret_cast<uint4*>(Ys + rr * G::LDK + cc) = keep_or_zero(x[i], live);
        } else {
          const Tin* kv = reinterpret_cast<const Tin*>(&kk);
          Tin y[VEC];
#pragma unroll
          for (int u = 0; u < VEC; ++u) y[u] = from_f32<Tin>(bk[i] * to_f32(kv[u]));
          *reinterpret_cast<uint4*>(Ys + rr * G::LDK + cc) = *reinterpret_cast<const uint4*>(y);
          if constexpr (kFused) {
            *reinterpret_cast<uint4*>(Xs + rr * G::LDK + cc) = kk;
          } else {
            *reinterpret_cast<uint4*>(Xs + rr * G::LDK + cc) = keep_or_zero(x[i], live);
          }
        }
      }
    }
    if constexpr (kDecay) {
      float* La = reinterpret_cast<float*>(smem + G::oLa);
#pragma unroll
      for (int i = 0; i < NLA; ++i) {
        const int e = tid + i * G::NT;
        if (e < C * DK / 4) {
          const int rr = e / (DK / 4), cc = (e % (DK / 4)) * 4;
          *reinterpret_cast<uint4*>(La + rr * G::LDA + cc) = keep_or_zero(la4[i], rr < vrows);
        }
      }
    }
    if constexpr (kFused) {
      float* gs = reinterpret_cast<float*>(smem + G::oGs);
      float* ds = reinterpret_cast<float*>(smem + G::oDs);
      float* rts = reinterpret_cast<float*>(smem + G::oRt);
      float* ras = reinterpret_cast<float*>(smem + G::oRa);
      if (tid < C) {
        gs[tid] = pg;
        rts[tid] = __expf(plp1 - plp);  // r_t = P_{t+1} / P_t
        ras[tid] = __expf(plp - plps);  // P_t / P_s <= 1
      }
      if (tid < DK) ds[tid] = pd;
    }
#pragma unroll
    for (int i = 0; i < NLV; ++i) {
      const int e = tid + i * G::NT;
      if (e < NVB) {
        const int rr = e / (DV / VEC), cc = (e % (DV / VEC)) * VEC;
        const uint4 vz = keep_or_zero(v[i], rr < vrows);
        const Tin* vv = reinterpret_cast<const Tin*>(&vz);
        Tin zz[VEC];
        if constexpr (kGdn2) {
          const Tin* ww = reinterpret_cast<const Tin*>(&w[i]);
#pragma unroll
          for (int u = 0; u < VEC; ++u) zz[u] = from_f32<Tin>(to_f32(ww[u]) * to_f32(vv[u]));
        } else {
#pragma unroll
          for (int u = 0; u < VEC; ++u) zz[u] = from_f32<Tin>(bv[i] * to_f32(vv[u]));
        }
        *reinterpret_cast<uint4*>(Zs + rr * G::LDV + cc) = *reinterpret_cast<const uint4*>(zz);
      }
    }
  }
};

// Persistent: workgroup g takes chunks g, g + gridDim.x, ... and fetches the
// next chunk's operands while the current one computes.
template <class V, int DK, int DV, int C, typename Tin>
__global__ __launch_bounds__(512) void wy_prep_kernel(ChunkArgs p, int nchunks,
                                                      WyBufs<Tin> wb) {
  using G = PrepCfg<V, DK, DV, C, Tin>;
  constexpr bool kGdn2 = std::is_same<V, Gdn2Variant>::value;
  constexpr bool kFused = kFusedVariant<V>;
  constexpr bool kDecay = kDecayVariant<V>;
  static_assert(!(kFused && kDecay) || G::kLaOwn,
                "the fused decay variant stages log alpha in a region of its own");
  constexpr int LDK = G::LDK, LDV = G::LDV, LDC = G::LDC, LDS16 = G::LDS16,
                TB = G::TB, DB = G::DB, VBT = G::VBT, NW = G::NW;
  __shared__ __attribute__((aligned(16))) unsigned char smem[G::bytes];
  Tin* Ys = reinterpret_cast<Tin*>(smem + G::oY);   // diag(rs) Y
  Tin* Xs = reinterpret_cast<Tin*>(smem + G::oX);
  Tin* Qs = reinterpret_cast<Tin*>(smem + G::oQ);   // Q (GDN-2: Q^ = gamma q)
  Tin* Zs = reinterpret_cast<Tin*>(smem + G::oZ);   // diag(rs) Z
  Tin* Ab = reinterpret_cast<Tin*>(smem + G::oAb);
  Tin* Tb = reinterpret_cast<Tin*>(smem + G::oTb);
  float* Am = reinterpret_cast<float*>(smem + G::oA);
  Tin* Ysc = reinterpret_cast<Tin*>(smem + G::oYs);
  float* gC = reinterpret_cast<float*>(smem + G::oG);

  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int total = p.B * p.H * nchunks;
  const Tin zero = from_f32<Tin>(0.f);

  // Blocks above the diagonal of T are zero (never written by the chunk
  // steps; GDN-2 restores them after its decay pass).
  for (int e = tid; e < C * C; e += G::NT) {
    const int rr = e / C, cc = e % C;
    if ((cc >> 4) > (rr >> 4)) Tb[rr * LDC + cc] = zero;
  }

  // Chunks are taken position-major, from the last position of every
  // (batch, head) down to the first: the scan that follows walks the chunks
  // from the first position up, so its first reads find the most recently
  // written operands still in the memory-side cache.
  const int BHn = total / nchunks;
  auto chunk_of = [&](int i) {
    const int jr = i / BHn, bh = i - jr * BHn;
    return bh * nchunks + (nchunks - 1 - jr);
  };
  PrepRegs<V, DK, DV, C, Tin> regs;
  if ((int)blockIdx.x < total) regs.load(p, chunk_of(blockIdx.x), nchunks);
  for (int pos = blockIdx.x; pos < total; pos += gridDim.x) {
    const int n = chunk_of(pos);
    regs.store(Ys, Xs, Qs, Zs, smem);
    // the next chunk's raw operands (the last chunk again at the end), in
    // three parts: the keys and queries here, the values and record after the
    // first barrier, the decays after the Gram section
    const int nn = chunk_of(min(pos + (int)gridDim.x, total - 1));
    regs.load_a(p, nn, nchunks);
    // Decay variants: lambda at the first and last token of each 16-token
    // block (doubling scratch), and, for this wave's diagonal tile when its
    // block decays too strongly for the factored form, the exact tile.
    float* Lsb = reinterpret_cast<float*>(smem + G::oYs);  // [TB][DK]
    float* Leb = Lsb + TB * DK;                             // [TB][DK]
    bool ex_diag = false;  // wave-uniform: this wave's diagonal tile is exact
    // workgroup-uniform: the whole chunk decays by at most e^-kExactDiag in
    // every channel, so factors relative to the chunk start stay finite
    // (read keys and queries times gamma_t <= 1, write keys over gamma_t
    // <= e^kExactDiag) and the per-tile factors of the block split are not
    // needed
    bool fast = true;
    auto decay_pass = [&]() {
      // Decay pass. (1) Column scan: TPC threads per channel c (lanes l and
      // l + 64/TPC of one wave), each over TPT consecutive tokens, turn the
      // staged log alpha into the inclusive prefix lambda in place and give
      // the exit decay g = gamma_C. (2) Block table and exact diagonals.
      // (3) Row pass, VEC channels per access, every factor <= 1:
      // X = x exp(lambda_e - lambda_t), Y = y exp(lambda_t - lambda_s),
      // Q = q exp(lambda_t - lambda_s) with s, e the first and last token of
      // t's block (GDN-2: x = k and y = b*k from the staged k and b; gated
      // OSDN: x = k~ and y = beta*k as staged).
      constexpr int TPC = G::TPC, TPT = G::TPT, CPW = 64 / TPC, LDA = G::LDA;
      float* La = reinterpret_cast<float*>(smem + G::oLa);
      __syncthreads();
      {
        const int c = wave * CPW + lane % CPW, part = lane / CPW;
        float lam[TPT];
        float run = 0.f;
#pragma unroll
        for (int m = 0; m < TPT; ++m) {
          run += La[(part * TPT + m) * LDA + c];
          lam[m] = run;
        }
        float incl = run;
#pragma unroll
        for (int d = 1; d < TPC; d <<= 1) {
          const float y = __shfl_up(incl, d * CPW, 64);
          if (part >= d) incl += y;
        }
        const float excl = incl - run;
        const float total_la = __shfl(incl, (TPC - 1) * CPW + lane % CPW, 64);
#pragma unroll
        for (int m = 0; m < TPT; ++m) La[(part * TPT + m) * LDA + c] = excl + lam[m];
        if (part == 0) gC[c] = __expf(total_la);
      }
      __syncthreads();
      {
        float m = 1.f;
        for (int c = lane; c < DK; c += 64) m = fminf(m, gC[c]);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) m = fminf(m, __shfl_xor(m, d, 64));
        fast = __builtin_amdgcn_readfirstlane(m >= __expf(-kExactDiag) ? 1 : 0) != 0;
      }
      if (!fast) {
        for (int e = tid; e < TB * DK; e += G::NT) {
          const int b = e / DK, c = e - b * DK;
          Lsb[e] = La[(16 * b) * LDA + c];
          Leb[e] = La[(16 * b + 15) * LDA + c];
        }
      }
      if (!fast && wave < TB) {
        // wave a owns diagonal tile a in the Gram step
        const int a = wave;
        float m = -1.f;
        for (int c = lane; c < DK; c += 64)
          m = fmaxf(m, La[(16 * a) * LDA + c] - La[(16 * a + 15) * LDA + c]);
        m = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max(m))));
        ex_diag = m > kExactDiag;
        if (ex_diag) {
          // the tile from the raw operands, exp(lambda_t - lambda_i) per
          // element, written where the Gram step would put it: A's block
          // transposed into the fp32 diagonal buffer, the scores (as P^T,
          // rows i, columns t) into the workspace
          const int gq = lane >> 4, cq = lane & 15;
          float* Ad = Am + a * 16 * G::LDD + cq * G::LDD + 4 * gq;
          Tin* pd = wb.pp + (size_t)n * C * C + (size_t)a * 16 * C;
#pragma unroll 1
          for (int r = 0; r < 4; ++r) {
            // A[t][i]: t = 4 gq + r, i = cq (strictly lower); P^T[i][t]:
            // i = 4 gq + r, t = cq (i <= t)
            const int tA = 16 * a + 4 * gq + r, iA = 16 * a + cq;
            const int iP = tA, tP = iA;
            float sa = 0.f, sp = 0.f;
#pragma unroll 1
            for (int c = 0; c < DK; ++c) {
              const float xi = to_f32(Xs[iA * LDK + c]), xp = to_f32(Xs[iP * LDK + c]);
              if (iA < tA) {
                float y = to_f32(Ys[tA * LDK + c]);
                if constexpr (kGdn2) y *= to_f32(Xs[tA * LDK + c]);
                sa += y * xi * __expf(La[tA * LDA + c] - La[iA * LDA + c]);
              }
              if (iP <= tP)
                sp += to_f32(Qs[tP * LDK + c]) * xp *
                      __expf(La[tP * LDA + c] - La[iP * LDA + c]);
            }
            Ad[r] = sa;
            Frag<C, Tin>::store_acc_elem(pd, a, r, sp);
          }
        }
      }
      __syncthreads();  // the row pass overwrites the raw operands
      constexpr int VEC = G::VEC;
      for (int item = tid; item < C * (DK / VEC); item += G::NT) {
        const int t = item / (DK / VEC), c0 = (item % (DK / VEC)) * VEC;
        const int tb = t >> 4;
        uint4 k4 = *reinterpret_cast<const uint4*>(Xs + t * LDK + c0);
        uint4 b4 = *reinterpret_cast<const uint4*>(Ys + t * LDK + c0);
        uint4 q4 = *reinterpret_cast<const uint4*>(Qs + t * LDK + c0);
        const Tin* kv = reinterpret_cast<const Tin*>(&k4);
        const Tin* bv = reinterpret_cast<const Tin*>(&b4);
        const Tin* qv = reinterpret_cast<const Tin*>(&q4);
        Tin xo[VEC], yo[VEC], qo[VEC];
#pragma unroll
        for (int u = 0; u < VEC; ++u) {
          const float lt = La[t * LDA + c0 + u];
          // relative to the chunk start (fast) or to t's block
          const float rs = fast ? 0.f : Lsb[tb * DK + c0 + u];
          const float re = fast ? 0.f : Leb[tb * DK + c0 + u];
          const float fs = __expf(lt - rs);  // <= 1
          const float fe = __expf(re - lt);  // <= 1 (block split), <= e^60 (fast)
          const float kk = to_f32(kv[u]);
          xo[u] = from_f32<Tin>(kk * fe);
          if constexpr (kGdn2)
            yo[u] = from_f32<Tin>(fs * to_f32(bv[u]) * kk);
          else
            yo[u] = from_f32<Tin>(fs * to_f32(bv[u]));
          qo[u] = from_f32<Tin>(fs * to_f32(qv[u]));
        }
        *reinterpret_cast<uint4*>(Xs + t * LDK + c0) = *reinterpret_cast<const uint4*>(xo);
        *reinterpret_cast<uint4*>(Ys + t * LDK + c0) = *reinterpret_cast<const uint4*>(yo);
        *reinterpret_cast<uint4*>(Qs + t * LDK + c0) = *reinterpret_cast<const uint4*>(qo);
      }
      if constexpr (G::kLaInGram) {
        __syncthreads();
        // the staging overlapped T: its blocks above the diagonal are zero
        // again
        for (int e = tid; e < C * C; e += G::NT) {
          const int rr = e / C, cc = e % C;
          if ((cc >> 4) > (rr >> 4)) Tb[rr * LDC + cc] = zero;
        }
      }
    };
    if constexpr (kDecay && !kFused) decay_pass();
    __syncthreads();
    regs.load_b(p, nn, nchunks);
    if constexpr (kFused) {
      // ---- K~ = d_t * k_t in place over the raw keys --------------------------
      // Inside the chunk the preconditioner follows its own recursion,
      // d_{t+1} = r_t d_t + g_t a_t (a_t = k_t * k_t), from the entry value.
      // One lane per (segment, channel pair): (A) the recursion over the
      // segment from zero, F_{t+1} = r_t F_t + g_t a_t, keeping F_t and k_t
      // of each token; (B) after a barrier, the segment's entry value from
      // those before it, d_s' = (P_s' / P_s) d_s + F_end(s) (factors <= 1),
      // then d_t = (P_t / P_s) d_s + F_t and K~_t = d_t * k_t.
      constexpr int NPR = DK / 2, SEGL = G::SEGL, NSEG = G::NSEG;
      using KP = KeyPairOf<Tin>;
      const float* gs = reinterpret_cast<const float*>(smem + G::oGs);
      const float* ds = reinterpret_cast<const float*>(smem + G::oDs);
      const float* rts = reinterpret_cast<const float*>(smem + G::oRt);
      const float* ras = reinterpret_cast<const float*>(smem + G::oRa);
      float* fe = reinterpret_cast<float*>(smem + G::oFe);
      const int pr = lane % NPR, seg = wave * (64 / NPR) + lane / NPR;
      const int s0 = seg * SEGL;
      typename KP::T kp[SEGL];
      float f0[SEGL], f1[SEGL];
      float F0 = 0.f, F1 = 0.f;
#pragma unroll
      for (int m = 0; m < SEGL; ++m) {
        const int t = s0 + m;
        kp[m] = *reinterpret_cast<const typename KP::T*>(Xs + t * LDK + 2 * pr);
        const float x0 = KP::lo(kp[m]), x1 = KP::hi(kp[m]);
        f0[m] = F0;
        f1[m] = F1;
        const float r = rts[t], g = gs[t];
        F0 = fmaf(r, F0, g * (x0 * x0));
        F1 = fmaf(r, F1, g * (x1 * x1));
      }
      *reinterpret_cast<float2*>(fe + seg * DK + 2 * pr) = float2{F0, F1};
      __syncthreads();
      float2 d = *reinterpret_cast<const float2*>(ds + 2 * pr);
#pragma unroll
      for (int v = 0; v + 1 < NSEG; ++v) {
        if (v < seg) {
          const int e1 = (v + 1) * SEGL - 1;  // last token of segment v
          const float rho = ras[e1] * rts[e1];
          const float2 fv = *reinterpret_cast<const float2*>(fe + v * DK + 2 * pr);
          d.x = fmaf(rho, d.x, fv.x);
          d.y = fmaf(rho, d.y, fv.y);
        }
      }
#pragma unroll
      for (int m = 0; m < SEGL; ++m) {
        const int t = s0 + m;
        const float ra = ras[t];
        *reinterpret_cast<typename KP::T*>(Xs + t * LDK + 2 * pr) =
            KP::pack(fmaf(ra, d.x, f0[m]) * KP::lo(kp[m]), fmaf(ra, d.y, f1[m]) * KP::hi(kp[m]));
      }
      __syncthreads();
      if constexpr (kDecay) {
        // the decay pass turns the preconditioned keys just formed into
        // K~/gamma (and decays the read keys and queries)
        decay_pass();
        __syncthreads();
      }
    }

    // ---- Gram A, scores P, diagonal blocks of T; X' fragments ---------------
    // Jobs: diagonal tile b on wave b, which then inverts its block; the
    // off-diagonal lower tiles (row-major order) on the other waves, so that
    // they run beside the serial inversions.
    {
      constexpr int NL = TB * (TB + 1) / 2;
      constexpr int NOFF = NL - TB;
      static_assert(NW > TB, "waves left for the off-diagonal tiles");
      constexpr int OW = NW - TB;
      const int njobs = wave < TB ? 1 : (NOFF - (wave - TB) + OW - 1) / OW;
      for (int it = 0; it < njobs; ++it) {
        const int job = wave < TB ? wave : TB + (wave - TB) + OW * it;
        int a, b;
        if (job < TB) {
          a = b = job;
        } else {
          int l = job - TB;
          a = 1;
          while (l >= a) { l -= a; ++a; }
          b = l;
        }
        Frag<DK, Tin> fy, fq, fx;
        fy.load(Ys + a * 16 * LDK, LDK);
        fq.load(Qs + a * 16 * LDK, LDK);
        fx.load(Xs + b * 16 * LDK, LDK);
        if constexpr (kDecay) {
          // block split: exp(lambda_{s_a} - lambda_{e_b}) per key channel
          // (exponent capped where an exact diagonal replaces the product
          // anyway)
          if (!fast) {
            const float* ls = Lsb + a * DK;
            const float* le = Leb + b * DK;
            scale_row_frag(fx, [&](int c) { return __expf(fminf(ls[c] - le[c], 80.f)); });
          }
        }
        // A tile (a, b); the scores as their transpose, tile (b, a) of
        // P^T = X Q^T, whose accumulator lanes hold exactly the scan's
        // permuted-order fragment of P's row block a, step b (stored
        // straight to the workspace; the mirrored tile above the diagonal
        // is stored as zeros)
        f32x4 aa = {0.f, 0.f, 0.f, 0.f}, pa = {0.f, 0.f, 0.f, 0.f};
        mma(pa, fx, fq);
        Tin* prow = wb.pp + (size_t)n * C * C;
        if (a > b) {
          // formed transposed (X Y^T), so that a lane holds four
          // consecutive columns of one row of A: one 8-byte LDS write
          mma(aa, fx, fy);
          Tin av[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) av[i] = from_f32<Tin>(aa[i]);
          *reinterpret_cast<RawQuad<Tin>*>(Ab + (a * 16 + acc_col()) * LDC + b * 16 + acc_row(0)) =
              *reinterpret_cast<const RawQuad<Tin>*>(av);
          Frag<C, Tin>::store_acc_tile(prow + (size_t)a * 16 * C, b, pa);
          Frag<C, Tin>::store_acc_tile(prow + (size_t)b * 16 * C, a,
                                       f32x4{0.f, 0.f, 0.f, 0.f});
        } else {
          mma(aa, fy, fx);
          float* Ad = Am + a * 16 * G::LDD;
          // (decay variants: a diagonal summed exactly in the decay pass is
          // already in place, in the buffer and in the workspace)
          bool from_mfma = true;
          if constexpr (kDecay) from_mfma = !ex_diag;
          if (from_mfma) {
            // diagonal tile: A in fp32, transposed, strictly lower part only
            float4 col;
            col.x = acc_row(0) > acc_col() ? aa[0] : 0.f;
            col.y = acc_row(1) > acc_col() ? aa[1] : 0.f;
            col.z = acc_row(2) > acc_col() ? aa[2] : 0.f;
            col.w = acc_row(3) > acc_col() ? aa[3] : 0.f;
            *reinterpret_cast<float4*>(Ad + acc_col() * G::LDD + acc_row(0)) = col;
            // P^T element (t' = row, t = column) kept where t' <= t
            f32x4 pm;
#pragma unroll
            for (int i = 0; i < 4; ++i) pm[i] = acc_row(i) <= acc_col() ? pa[i] : 0.f;
            Frag<C, Tin>::store_acc_tile(prow + (size_t)a * 16 * C, a, pm);
          }
          // T's diagonal block by forward substitution: lane c < 16 owns
          // column c; pending sums are updated as soon as each entry is final.
          wave_lds_sync();
          if (lane < 16) {
            const int c = lane;
            float x[16], sv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) sv[i] = (i == c) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
              x[m] = sv[m];
              float cv[16];
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4) {
                const float4 v4 = *reinterpret_cast<const float4*>(Ad + m * G::LDD + 4 * q4);
                cv[4 * q4] = v4.x; cv[4 * q4 + 1] = v4.y;
                cv[4 * q4 + 2] = v4.z; cv[4 * q4 + 3] = v4.w;
              }
#pragma unroll
              for (int i = m + 1; i < 16; ++i) sv[i] -= cv[i] * x[m];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i)
              Tb[(a * 16 + i) * LDC + a * 16 + c] = from_f32<Tin>(x[i]);
          }
        }
      }
      // X' = X diag(g) as k-major fragments, one channel block per job
      // (loops that store have a static trip count, so that the compiler can
      // count the stores and the next chunk's fetch is not waited on early)
      const size_t xoff = (size_t)n * C * DK;
#pragma unroll
      for (int it = 0; it < (DB + NW - 1) / NW; ++it) {
        const int db = wave + it * NW;
        if (db >= DB) break;
        Frag<C, Tin> fx;
        fx.load_kmajor_perm(Xs + db * 16, LDK);  // the scan's k order
        if constexpr (kDecay) {
          // exit keys x_i gamma_C / gamma_i = X_i gamma_C (fast), or
          // X_i exp(lambda_C - lambda_{e_b}) (block split)
          const int c = db * 16 + (lane & 15);
          if (fast) {
            const float gc = gC[c];
            scale_kperm_frag(fx, [&](int) { return gc; });
          } else {
            float fb[TB];
#pragma unroll
            for (int b2 = 0; b2 < TB; ++b2)
              fb[b2] = __expf(Leb[(TB - 1) * DK + c] - Leb[b2 * DK + c]);
            scale_kperm_frag(fx, [&](int t) { return fb[t >> 4]; });
          }
        }
        fx.store_global(wb.xp + xoff + (size_t)db * 16 * C);
      }
      if constexpr (kDecay) {
        if (tid < DK) wb.g[(size_t)n * DK + tid] = gC[tid];
      }
    }
    __syncthreads();
    regs.load_c(p, nn, nchunks);
    if (kDecay && !fast) {
      // read keys and queries relative to the chunk start from here on (for
      // Wk and the decayed queries): times exp(lambda_{s_b}) <= 1
      constexpr int VEC = G::VEC;
      for (int item = tid; item < C * (DK / VEC); item += G::NT) {
        const int t = item / (DK / VEC), c0 = (item % (DK / VEC)) * VEC;
        const float* ls = Lsb + (t >> 4) * DK + c0;
        uint4 y4 = *reinterpret_cast<const uint4*>(Ys + t * LDK + c0);
        uint4 q4 = *reinterpret_cast<const uint4*>(Qs + t * LDK + c0);
        Tin* yv = reinterpret_cast<Tin*>(&y4);
        Tin* qv = reinterpret_cast<Tin*>(&q4);
#pragma unroll
        for (int u = 0; u < VEC; ++u) {
          const float f = __expf(ls[u]);
          yv[u] = from_f32<Tin>(f * to_f32(yv[u]));
          qv[u] = from_f32<Tin>(f * to_f32(qv[u]));
        }
        *reinterpret_cast<uint4*>(Ys + t * LDK + c0) = y4;
        *reinterpret_cast<uint4*>(Qs + t * LDK + c0) = q4;
      }
      __syncthreads();  // the doubling overwrites the block table
    }


    // ---- recursive doubling, T21 = -T22 (A21 T11) ----------------------------
    // One job = one 16-wide column of T21 in one pair: that column of
    // Y = A21 T11 goes to the wave's own scratch (row-major), then the same
    // column of T21 = -T22 Y; the right operands are read k-major. Both
    // products are formed transposed, so that a lane writes four
    // consecutive columns of one row with one 8-byte access.
    {
      Tin* ys = Ysc + wave * (C / 2) * LDS16;
#pragma unroll
      for (int s = 16; s < C; s *= 2) {
        const int nt = s / 16;
        const int jobs = (C / (2 * s)) * nt;
        for (int job = wave; job < jobs; job += NW) {
          const int pp = job / nt, c = job % nt;
          const int rb = 2 * s * pp + s, cb = 2 * s * pp;
          for (int r = 0; r < nt; ++r) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int kk = 0; kk < s; kk += 16) {
              Frag<16, Tin> fa, fb;
              fa.load(Ab + (rb + r * 16) * LDC + cb + kk, LDC);
              fb.load_kmajor(Tb + (cb + kk) * LDC + cb + c * 16, LDC);
              mma(acc, fb, fa);
            }
            Tin yv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) yv[i] = from_f32<Tin>(acc[i]);
            *reinterpret_cast<RawQuad<Tin>*>(ys + (r * 16 + acc_col()) * LDS16 + acc_row(0)) =
                *reinterpret_cast<const RawQuad<Tin>*>(yv);
          }
          wave_lds_sync();
          for (int r = 0; r < nt; ++r) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int kk = 0; kk < s; kk += 16) {
              Frag<16, Tin> fa, fb;
              fa.load(Tb + (rb + r * 16) * LDC + rb + kk, LDC);
              fb.load_kmajor(ys + kk * LDS16, LDS16);
              mma(acc, fb, fa);
            }
            Tin tv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) tv[i] = from_f32<Tin>(-acc[i]);
            *reinterpret_cast<RawQuad<Tin>*>(Tb + (rb + r * 16 + acc_col()) * LDC + cb + c * 16 +
                                             acc_row(0)) =
                *reinterpret_cast<const RawQuad<Tin>*>(tv);
          }
          wave_lds_sync();  // the scratch is rewritten by this wave's next job
        }
        __syncthreads();
      }
    }

    // ---- Wk = T diag(rs) Y and U = T diag(rs) Z --------------------------------
    // One job = one 16-wide column block of Y (or Z), all row blocks. Both go
    // from the accumulators straight to the workspace: Wk formed transposed,
    // so that a lane's four consecutive columns of one row are one piece of
    // the scan's row-block fragment; U as accumulator tiles.
    const size_t uoff = (size_t)n * C * DV;
    const size_t koff = (size_t)n * C * DK;
    {
      Frag<C, Tin> ft[TB];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) ft[tb].load(Tb + tb * 16 * LDC, LDC);
#pragma unroll
      for (int it = 0; it < (DB + VBT + NW - 1) / NW; ++it) {
        const int job = wave + it * NW;
        if (job >= DB + VBT) break;
        const bool isU = job >= DB;
        const int ct = isU ? job - DB : job;
        Tin* M = isU ? Zs : Ys;
        const int ld = isU ? LDV : LDK;
        Frag<C, Tin> fm;
        fm.load_kmajor(M + ct * 16, ld);
        f32x4 acc[TB];
        if (isU) {
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) {
            acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
            mma(acc[tb], ft[tb], fm);
          }
#pragma unroll
          for (int tb = 0; tb < TB; ++tb)
            RawTile<Tin>::store(acc[tb], wb.u + uoff + u_tile(tb, ct, VBT));
        } else {
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) {
            acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
            mma(acc[tb], fm, ft[tb]);
          }
#pragma unroll
          for (int tb = 0; tb < TB; ++tb)
            Frag<DK, Tin>::store_acc_kblock(wb.wk + koff + (size_t)tb * 16 * DK, ct, acc[tb]);
        }
      }
    }

    // ---- decay variants: the decayed queries Q^ as row-block fragments ------
    if constexpr (kDecay) {
#pragma unroll
      for (int it = 0; it < (TB + NW - 1) / NW; ++it) {
        const int tb = wave + it * NW;
        if (tb >= TB) break;
        Frag<DK, Tin> f;
        f.load(Qs + tb * 16 * LDK, LDK);
        f.store_global(wb.qh + koff + (size_t)tb * 16 * DK);
      }
    }
    __syncthreads();  // the next chunk's operands overwrite the tiles
  }
}

// ---------------------------------------------------------------------------
// scan
// ---------------------------------------------------------------------------
template <int DK, int C, int VT, typename Tin>
struct ScanCfg {
  static constexpr int NW = 4, NT = 256;
  static constexpr int PAD = sizeof(Tin) == 2 ? 8 : 4;
  static constexpr int LDK = DK + PAD, LDW = C + PAD, LDO = VT + PAD;
  static constexpr int TB = C / 16, VB = VT / 16, DB = DK / 16;
  static constexpr size_t E = sizeof(Tin);
  static constexpr size_t oS = 0;                                 // state copy [VT][Dk]
  static constexpr size_t oW = oS + (size_t)VT * LDK * E;        // W^T [VT][C]
  static constexpr size_t oO = oW + (size_t)VT * LDW * E;        // output rows [C][VT]
  static constexpr size_t bytes = oO + (size_t)C * LDO * E;
  // State tiles per wave: every value tile times a contiguous run of DPW
  // channel tiles.
  static constexpr int DPW = (DB + NW - 1) / NW;
  static constexpr int NS = VB * DPW;
  static_assert(TB <= NW, "one row block per wave");
};

// DECAY: the chunk operands carry a decay (decayed queries Q^ and exit
// decays g read from the workspace); KD: the state is stored [Dk, Dv].
template <bool DECAY, int DK, int C, int VT, typename Tin>
struct ScanRegs {
  using G = ScanCfg<DK, C, VT, Tin>;
  Frag<DK, Tin> wk, qh;      // the wave's 16 rows of Wk and of the queries
  Frag<C, Tin> pr;           // the same rows of the scores P
  RawTile<Tin> u[G::VB];
  Frag<C, Tin> x[G::DPW];
  float4 gd[G::DPW];         // exit decays of the lane's four state channels

  // Chunk j of (batch, head) bh. Loads are unconditional (indices of idle
  // waves and rows past the sequence end clamped into range), so that the
  // compiler can count them and a prefetch is only waited on where its data
  // is used.
  __device__ __forceinline__ void load(const WyBufs<Tin>& wb, const Tin* q, int bh,
                                       int j, int nchunks, int T, int Dv, int vt,
                                       int wave) {
    constexpr int VB = G::VB;
    const int VBT = Dv / 16;
    const int tb = min(wave, G::TB - 1);
    const size_t n = (size_t)bh * nchunks + j;
    const size_t koff = n * C * DK + (size_t)tb * 16 * DK;
    wk.load_global(wb.wk + koff);
    if constexpr (DECAY) {
      qh.load_global(wb.qh + koff);
    } else {
      const int row = min(tb * 16 + (int)(threadIdx.x & 15), min(C, T - j * C) - 1);
      qh.load_row(q + ((size_t)bh * T + (size_t)j * C + row) * DK);
    }
    if constexpr (sizeof(Tin) == 2 && C % 32 == 0) {
      // P is zero right of its diagonal blocks. Its columns (tokens) are in
      // the permuted slot order of W^T: piece i holds token tiles 2i and
      // 2i + 1, so a piece is zero for row blocks below tile 2i. Such a
      // piece is read from piece 0's addresses instead (so that it touches
      // no further memory); the step zeroes it where P is used.
      const int lane = threadIdx.x & 63;
      const Tin* pb = wb.pp + n * C * C + (size_t)tb * 16 * C;
#pragma unroll
      for (int i = 0; i < C / 32; ++i) {
        const int src = 2 * i <= tb ? i * 64 + lane : lane;
        pr.v[i] = *reinterpret_cast<const bf16x8*>(pb + src * 8);
      }
    } else {
      pr.load_global(wb.pp + n * C * C + (size_t)tb * 16 * C);
    }
    const Tin* ub = wb.u + n * C * Dv;
    if constexpr (VB % 2 == 0) {
#pragma unroll
      for (int pr2 = 0; pr2 < VB / 2; ++pr2)
        RawTile<Tin>::load_pair(ub + u_tile(tb, vt * VB + 2 * pr2, VBT), u[2 * pr2],
                                u[2 * pr2 + 1]);
    } else {
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) u[vb].load(ub + u_tile(tb, vt * VB + vb, VBT));
    }
#pragma unroll
    for (int d = 0; d < G::DPW; ++d) {
      const int db = min(wave * G::DPW + d, G::DB - 1);
      x[d].load_global(wb.xp + n * C * DK + (size_t)db * 16 * C);
      if constexpr (DECAY)
        gd[d] = *reinterpret_cast<const float4*>(wb.g + n * DK + db * 16 +
                                                 4 * ((threadIdx.x & 63) >> 4));
    }
  }
};

template <bool DECAY, bool KD, int DK, int C, int VT, typename Tin>
__global__ __launch_bounds__(256) void wy_scan_kernel(ChunkArgs p, int nchunks,
                                                      WyBufs<Tin> wb) {
  using G = ScanCfg<DK, C, VT, Tin>;
  using R = ScanRegs<DECAY, DK, C, VT, Tin>;
  constexpr int LDK = G::LDK, LDW = G::LDW, LDO = G::LDO, TB = G::TB, VB = G::VB,
                DB = G::DB, DPW = G::DPW;
  __shared__ __attribute__((aligned(16))) unsigned char smem[G::bytes];
  Tin* Ss = reinterpret_cast<Tin*>(smem + G::oS);   // state copy [v][dk]
  Tin* Wt = reinterpret_cast<Tin*>(smem + G::oW);   // W^T [v][token]
  Tin* Os = reinterpret_cast<Tin*>(smem + G::oO);   // output rows [t][v]

  const int T = p.T, Dv = p.Dv;
  const int nvt = Dv / VT;
  // XCD-aware numbering: workgroups go round-robin over the 8 XCDs; keep all
  // value tiles of one (batch, head) on one XCD so they share its L2.
  int lin = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) lin = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int bh = lin / nvt, vt = lin - bh * nvt;
  const int wave = wave_id();
  const int v0 = vt * VT;
  Tin* o = (Tin*)p.o;
  const Tin* q = (const Tin*)p.q;

  // Persistent state slice S[v][dk] (v in this tile), fp32, MFMA layout.
  // OSDN stores the state [Dv][Dk]; GDN-2 stores it [Dk][Dv].
  auto sidx = [&](int vv, int kk) -> size_t {
    return KD ? ((size_t)bh * DK + kk) * Dv + v0 + vv
                : ((size_t)bh * Dv + v0 + vv) * DK + kk;
  };
  // The state tiles are held transposed: lane element i of tile (vb, db) is
  // S[v = vb*16 + acc_col()][dk = db*16 + acc_row(i)], so that each lane's
  // four values are consecutive channels of one row of the bf16 copy in LDS
  // (one 8-byte write).
  f32x4 Sacc[G::NS];
  auto store_state = [&](const f32x4& acc, int vb, int db) {
    Tin sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = from_f32<Tin>(acc[i]);
    *reinterpret_cast<RawQuad<Tin>*>(Ss + (vb * 16 + acc_col()) * LDK + db * 16 + acc_row(0)) =
        *reinterpret_cast<const RawQuad<Tin>*>(sv);
  };
#pragma unroll
  for (int vb = 0; vb < VB; ++vb) {
#pragma unroll
    for (int d = 0; d < DPW; ++d) {
      const int db = wave * DPW + d;
      f32x4& acc = Sacc[vb * DPW + d];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = 0.f;
        if (db < DB && p.S0) x = p.S0[sidx(vb * 16 + acc_col(), db * 16 + acc_row(i))];
        acc[i] = x;
      }
      if (db < DB) store_state(acc, vb, db);
    }
  }
  __syncthreads();

  // One chunk step; TAIL: the chunk may be partial (rows past T are not
  // stored). `cur` holds chunk j (fetched during the previous step); chunk
  // j + 1 is fetched into `fetch` at the start (the last chunk again on the
  // final step, so that every step issues the same loads). Guards that
  // always hold for the tile configuration fold away at compile time.
  constexpr bool kAllRowWaves = TB == G::NW, kAllColWaves = DPW * G::NW == DB;
  auto step = [&](int j, auto tail, R& fetch, const R& cur) {
    constexpr bool TAIL = decltype(tail)::value;
    const size_t t0 = (size_t)bh * T + (size_t)j * C;
    const int valid = min(C, T - j * C);
    fetch.load(wb, q, bh, min(j + 1, nchunks - 1), nchunks, T, Dv, vt, wave);
    // ---- W = U - Wk S0^T (to LDS, transposed) and Q S0^T ------------------
    // A lane's four W values (tokens 4g..4g+3 of one column) are contiguous
    // in W^T.
    f32x4 oacc[VB];
    if (kAllRowWaves || wave < TB) {
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        Frag<DK, Tin> fs;
        fs.load(Ss + vb * 16 * LDK, LDK);
        f32x4 wa = {0.f, 0.f, 0.f, 0.f};
        oacc[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
        mma(wa, cur.wk, fs);
        mma(oacc[vb], fs, cur.qh);  // transposed: [v][t]
        Tin w4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w4[i] = from_f32<Tin>(cur.u[vb][i] - wa[i]);
        typedef __attribute__((ext_vector_type(4))) unsigned short u16x4;
        if constexpr (sizeof(Tin) == 2) {
          // bf16: the four tokens go to their slots of the permuted order
          // (tile tb fills half tb % 2 of 32-wide step tb / 2), so that the
          // fragments below are plain 16-byte row reads
          const int g = (threadIdx.x & 63) >> 4;
          const int slot = (wave >> 1) < C / 32 ? 32 * (wave >> 1) + 8 * g + 4 * (wave & 1)
                                                : 32 * (C / 32) + 4 * g;
          *reinterpret_cast<u16x4*>(Wt + (vb * 16 + acc_col()) * LDW + slot) =
              *reinterpret_cast<const u16x4*>(w4);
        } else
          *reinterpret_cast<float4*>(Wt + (vb * 16 + acc_col()) * LDW + wave * 16 + acc_row(0)) =
              *reinterpret_cast<const float4*>(w4);
      }
    }
    __syncthreads();
    // ---- O = scale (Q S0^T + P W); S = S diag(g) + W^T X' -------------------
    {
      Frag<C, Tin> fw[VB];
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        if constexpr (sizeof(Tin) == 2)
          fw[vb].load(Wt + vb * 16 * LDW, LDW);       // stored in slot order
        else
          fw[vb].load_perm(Wt + vb * 16 * LDW, LDW);
      }
      if (kAllRowWaves || wave < TB) {
        // the wave's 16 output rows go through LDS (rows of this wave only)
        // and out as one 16-byte store per lane
        Frag<C, Tin> prz = cur.pr;
        if constexpr (sizeof(Tin) == 2 && C % 32 == 0) {
          // the pieces of P that the operand fetch skipped (zero in P)
          const int tb = min(wave, TB - 1);
#pragma unroll
          for (int i = 0; i < C / 32; ++i)
            if (2 * i > tb) prz.v[i] = bf16x8{};
        }
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
          mma(oacc[vb], fw[vb], prz);  // transposed: four columns per lane
          Tin ov[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) ov[i] = from_f32<Tin>(p.scale * oacc[vb][i]);
          *reinterpret_cast<RawQuad<Tin>*>(Os + (wave * 16 + acc_col()) * LDO + vb * 16 +
                                           acc_row(0)) =
              *reinterpret_cast<const RawQuad<Tin>*>(ov);
        }
        wave_lds_sync();
        constexpr int VPL = 16 / (int)sizeof(Tin);           // elements per lane access
        constexpr int LPR = VT / VPL;                        // lanes per row
        constexpr int RPI = 64 / LPR;                        // rows per access
#pragma unroll
        for (int r0 = 0; r0 < 16; r0 += RPI) {
          const int rr = wave * 16 + r0 + (threadIdx.x & 63) / LPR;
          const int cc = ((threadIdx.x & 63) % LPR) * VPL;
          if (r0 + (threadIdx.x & 63) / LPR < 16 && (!TAIL || rr < valid))
            *reinterpret_cast<u32x4*>(o + (t0 + rr) * Dv + v0 + cc) =
                *reinterpret_cast<const u32x4*>(Os + rr * LDO + cc);
        }
      }
#pragma unroll
      for (int d = 0; d < DPW; ++d) {
        const int db = wave * DPW + d;
        if (kAllColWaves || db < DB) {
#pragma unroll
          for (int vb = 0; vb < VB; ++vb) {
            f32x4& acc = Sacc[vb * DPW + d];
            if constexpr (DECAY) {
              acc[0] *= cur.gd[d].x;
              acc[1] *= cur.gd[d].y;
              acc[2] *= cur.gd[d].z;
              acc[3] *= cur.gd[d].w;
            }
            mma(acc, cur.x[d], fw[vb]);  // transposed state tile
            store_state(acc, vb, db);
          }
        }
      }
    }
    __syncthreads();
  };

  // Two register sets in turn (even steps fetch into rb and use ra, odd
  // steps the reverse), unrolled so that each set is a fixed object.
  R ra, rb;
  if (nchunks > 0) ra.load(wb, q, bh, 0, nchunks, T, Dv, vt, wave);
  using Full = std::false_type;
  using Tail = std::true_type;
  const int nfull = T / C;  // chunks with C valid rows
  int j = 0;
  for (; j + 1 < nfull; j += 2) {
    step(j, Full{}, rb, ra);
    step(j + 1, Full{}, ra, rb);
  }
  if (j < nfull) {
    step(j, Full{}, rb, ra);  // j even
    ++j;
  }
  if (j < nchunks) {
    if ((j & 1) == 0)
      step(j, Tail{}, rb, ra);
    else
      step(j, Tail{}, ra, rb);
  }

  if (p.ST) {
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
#pragma unroll
      for (int d = 0; d < DPW; ++d) {
        const int db = wave * DPW + d;
        if (db < DB) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            p.ST[sidx(vb * 16 + acc_col(), db * 16 + acc_row(i))] = Sacc[vb * DPW + d][i];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------
// Resident prep workgroups per compute unit (LDS-limited).
template <class V, int DK, int DV, int C, typename Tin>
constexpr int kPrepWgPerCu() {
  return (int)(163840 / PrepCfg<V, DK, DV, C, Tin>::bytes) < 2
             ? 1
             : (int)(163840 / PrepCfg<V, DK, DV, C, Tin>::bytes);
}

// Value-tile width of the scan: 32 columns when that already gives one
// workgroup per compute unit (256 CUs), else 16 for more parallelism.
static int pick_vt(int BH, int Dv) { return (BH * (Dv / 32) >= 256) ? 32 : 16; }

template <class V, int DK, int DV, int C, typename Tin>
static int launch_cfg(const ChunkArgs& a, hipStream_t s) {
  if constexpr (!PrepCfg<V, DK, DV, C, Tin>::fits) {
    return -1;
  } else {
    constexpr bool kGdn2 = std::is_same<V, Gdn2Variant>::value;
    constexpr bool kGated = std::is_same<V, OsdnGatedVariant>::value ||
                            std::is_same<V, OsdnGatedFusedVariant>::value;
    constexpr bool kDecay = kDecayVariant<V>;
    const int BH = a.B * a.H, nch = (a.T + C - 1) / C;
    if (BH == 0) return 0;
    const WyBufs<Tin> wb = wy_bufs<Tin>(a.ws, BH, nch, C, DK, DV, kDecay);
    if (nch > 0) {
      // persistent grid: a few workgroups per compute unit at most
      const int grid = std::min(BH * nch, 256 * kPrepWgPerCu<V, DK, DV, C, Tin>());
      const int tk_prep = ktimer_before(s, kGdn2    ? "gdn2_prep"
                       : std::is_same<V, OsdnGatedFusedVariant>::value ? "gated_prep_fused"
                       : kGated ? "gated_prep"
                       : std::is_same<V, OsdnFusedVariant>::value ? "wy_prep_fused"
                                                                  : "wy_prep");
      hipLaunchKernelGGL((wy_prep_kernel<V, DK, DV, C, Tin>), dim3(grid),
                         dim3(512), 0, s, a, nch, wb);
      ktimer_after(s, tk_prep);
      const int rc = (int)hipGetLastError();
      if (rc) return rc;
    }
    const int tk_scan = ktimer_before(s, kGdn2 ? "gdn2_scan" : kGated ? "gated_scan" : "wy_scan");
    if (pick_vt(BH, DV) == 32)
      hipLaunchKernelGGL((wy_scan_kernel<kDecay, kGdn2, DK, C, 32, Tin>),
                         dim3(BH * (DV / 32)), dim3(256), 0, s, a, nch, wb);
    else
      hipLaunchKernelGGL((wy_scan_kernel<kDecay, kGdn2, DK, C, 16, Tin>),
                         dim3(BH * (DV / 16)), dim3(256), 0, s, a, nch, wb);
    ktimer_after(s, tk_scan);
    return (int)hipGetLastError();
  }
}

template <class V, int DK, int DV, typename Tin>
static int launch_dv(const ChunkArgs& a, hipStream_t s) {
  if constexpr (kFusedVariant<V>) {
    return a.chunk == kPrecondChunk ? launch_cfg<V, DK, DV, kPrecondChunk, Tin>(a, s)
                                    : -1;
  }
  switch (a.chunk) {
    case 16: return launch_cfg<V, DK, DV, 16, Tin>(a, s);
    case 32: return launch_cfg<V, DK, DV, 32, Tin>(a, s);
    case 64: return launch_cfg<V, DK, DV, 64, Tin>(a, s);
  }
  return -1;
}

template <class V, int DK, typename Tin>
static int launch_dk(const ChunkArgs& a, hipStream_t s) {
  switch (a.Dv) {
    case 32: return launch_dv<V, DK, 32, Tin>(a, s);
    case 64: return launch_dv<V, DK, 64, Tin>(a, s);
    case 128: return launch_dv<V, DK, 128, Tin>(a, s);
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

int launch_osdn_gated_chunk(const ChunkArgs& a, hipStream_t s) {
  return launch_variant<OsdnGatedVariant>(a, s);
}

int launch_osdn_gated_fused(const ChunkArgs& a, hipStream_t s) {
  if (a.chunk != kPrecondChunk) return -1;
  return launch_variant<OsdnGatedFusedVariant>(a, s);
}

int launch_osdn_fused(const ChunkArgs& a, hipStream_t s) {
  if (a.chunk != kPrecondChunk) return -1;
  return launch_variant<OsdnFusedVariant>(a, s);
}

// Supported sizes: those where the largest layout (fused OSDN) fits, for
// every variant alike.
template <int DK, int DV, typename Tin>
static bool fits_dv(int chunk) {
  switch (chunk) {
    case 16: return PrepCfg<OsdnFusedVariant, DK, DV, 16, Tin>::fits;
    case 32: return PrepCfg<OsdnFusedVariant, DK, DV, 32, Tin>::fits;
    case 64: return PrepCfg<OsdnFusedVariant, DK, DV, 64, Tin>::fits;
  }
  return false;
}

template <int DK, typename Tin>
static bool fits_dk(int Dv, int chunk) {
  switch (Dv) {
    case 32: return fits_dv<DK, 32, Tin>(chunk);
    case 64: return fits_dv<DK, 64, Tin>(chunk);
    case 128: return fits_dv<DK, 128, Tin>(chunk);
  }
  return false;
}

template <int DK, typename Tin>
static bool gated_fused_fits(int Dv) {
  switch (Dv) {
    case 32: return PrepCfg<OsdnGatedFusedVariant, DK, 32, kPrecondChunk, Tin>::fits;
    case 64: return PrepCfg<OsdnGatedFusedVariant, DK, 64, kPrecondChunk, Tin>::fits;
    case 128: return PrepCfg<OsdnGatedFusedVariant, DK, 128, kPrecondChunk, Tin>::fits;
  }
  return false;
}

bool gated_fused_supported(int Dk, int Dv, int bf16) {
  if (bf16) {
    switch (Dk) {
      case 32: return gated_fused_fits<32, __bf16>(Dv);
      case 64: return gated_fused_fits<64, __bf16>(Dv);
      case 128: return gated_fused_fits<128, __bf16>(Dv);
    }
  } else {
    switch (Dk) {
      case 32: return gated_fused_fits<32, float>(Dv);
      case 64: return gated_fused_fits<64, float>(Dv);
      case 128: return gated_fused_fits<128, float>(Dv);
    }
  }
  return false;
}

bool osdn_chunk_supported(int Dk, int Dv, int chunk, int bf16) {
  if (bf16) {
    switch (Dk) {
      case 32: return fits_dk<32, __bf16>(Dv, chunk);
      case 64: return fits_dk<64, __bf16>(Dv, chunk);
      case 128: return fits_dk<128, __bf16>(Dv, chunk);
    }
  } else {
    switch (Dk) {
      case 32: return fits_dk<32, float>(Dv, chunk);
      case 64: return fits_dk<64, float>(Dv, chunk);
      case 128: return fits_dk<128, float>(Dv, chunk);
    }
  }
  return false;
}

// The GDN-2 decay pass splits each chunk's tokens over 512/Dk threads per
// channel, so the chunk must hold at least that many tokens.
bool gdn2_chunk_supported(int Dk, int Dv, int chunk, int bf16) {
  return osdn_chunk_supported(Dk, Dv, chunk, bf16) && chunk >= 512 / Dk;
}

}  // namespace osdn
