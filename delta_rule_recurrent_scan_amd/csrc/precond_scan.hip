// Phase 1 of the OSDN forward: the preconditioner scan over the key stream.
//
// [OSDN-it] section 2.2 (two-phase implementation, first phase) and 2.3:
// per (batch, head), for t = 1..T
//   a = k_t*k_t, n = ||k_t||^2, c = <d_t, a>, k~_t = d_t * k_t,
//   g = eta beta_t (1 - beta_t c) / n   (0 when n = 0),
//   d_{t+1} = r_t d_t + g a            (descent on the closed-form surrogate).
// The scan reads only k, beta, r, eta and d0, so it runs before, and
// independently of, the memory update.
//
// Token-serial form: one wave per (batch, head); lane l owns channels
// [l*CPL, l*CPL + CPL). The per-token dot product <d_t, a> is a wave-wide
// reduction in DPP and cross-row swaps. Keys are loaded a block of tokens
// ahead so that memory latency stays off the serial chain.
#include "device_common.hpp"
#include "launch.hpp"

namespace osdn {

template <int DK, typename Tin>
struct KeyVec {
  static constexpr int CPL = DK >= 64 ? DK / 64 : 1;
  float x[CPL];
};

template <int DK, typename Tin>
__device__ __forceinline__ void load_key(KeyVec<DK, Tin>& kv, const Tin* row,
                                         int lane) {
  constexpr int CPL = KeyVec<DK, Tin>::CPL;
  if (DK >= 64 || lane < DK) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) kv.x[j] = to_f32(row[lane * CPL + j]);
  } else {
#pragma unroll
    for (int j = 0; j < CPL; ++j) kv.x[j] = 0.f;
  }
}

template <int DK, typename Tin, int TB>
__global__ __launch_bounds__(64) void precond_scan_serial_kernel(
    int T, const Tin* __restrict__ k, const float* __restrict__ beta,
    const float* __restrict__ r, float eta, const float* __restrict__ d0,
    Tin* __restrict__ ktil, float* __restrict__ dT) {
  constexpr int CPL = KeyVec<DK, Tin>::CPL;
  const int bh = blockIdx.x;
  const int lane = threadIdx.x;
  const bool active = DK >= 64 || lane < DK;
  const size_t base = (size_t)bh * T;
  const Tin* kp = k + base * DK;
  Tin* kt = ktil ? ktil + base * DK : nullptr;
  const float* bp = beta + base;
  const float* rp = r ? r + base : nullptr;

  float d[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j)
    d[j] = active ? (d0 ? d0[(size_t)bh * DK + lane * CPL + j] : 1.f) : 0.f;

  KeyVec<DK, Tin> cur[TB], nxt[TB];
  float bcur[TB], rcur[TB], bnxt[TB], rnxt[TB];
  auto load_block = [&](int t0, KeyVec<DK, Tin>* kv, float* bb, float* rr) {
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      const int t = t0 + i;
      if (t < T) {
        load_key<DK, Tin>(kv[i], kp + (size_t)t * DK, lane);
        bb[i] = bp[t];
        rr[i] = rp ? rp[t] : 1.f;
      } else {
#pragma unroll
        for (int j = 0; j < CPL; ++j) kv[i].x[j] = 0.f;
        bb[i] = 0.f;
        rr[i] = 1.f;
      }
    }
  };

  load_block(0, cur, bcur, rcur);
  for (int t0 = 0; t0 < T; t0 += TB) {
    load_block(t0 + TB, nxt, bnxt, rnxt);
    // Key norms and step scales of the block do not depend on d: compute them
    // first, as independent reductions.
    float e[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) s += cur[i].x[j] * cur[i].x[j];
      const float n = wave_sum(s);
      e[i] = n > 0.f ? eta * bcur[i] / n : 0.f;
    }
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      const int t = t0 + i;
      if (t >= T) break;
      float a[CPL], s = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        a[j] = cur[i].x[j] * cur[i].x[j];
        s += d[j] * a[j];
      }
      const float c = wave_sum(s);
      if (active && kt) {
#pragma unroll
        for (int j = 0; j < CPL; ++j)
          kt[(size_t)t * DK + lane * CPL + j] = from_f32<Tin>(d[j] * cur[i].x[j]);
      }
      const float g = e[i] * (1.f - bcur[i] * c);
#pragma unroll
      for (int j = 0; j < CPL; ++j) d[j] = rcur[i] * d[j] + g * a[j];
    }
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      cur[i] = nxt[i];
      bcur[i] = bnxt[i];
      rcur[i] = rnxt[i];
    }
  }
  if (dT && active) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) dT[(size_t)bh * DK + lane * CPL + j] = d[j];
  }
}

template <int DK, typename Tin>
static int launch_dk(const PrecondArgs& a, hipStream_t s) {
  dim3 grid(a.B * a.H), block(64);
  hipLaunchKernelGGL((precond_scan_serial_kernel<DK, Tin, 8>), grid, block, 0,
                     s, a.T, (const Tin*)a.k, a.beta, a.r, a.eta, a.d0,
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
