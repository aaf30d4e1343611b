// C ABI of libosdn.so: host-side validation, workspace sizing and the launch
// sequence. Declarations and the full contract are in include/osdn.h.
#include "../../include/osdn.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace {

bool dim_ok(int d) { return d == 32 || d == 64 || d == 128; }
bool chunk_ok(int c) { return c == 16 || c == 32 || c == 64; }
size_t elem(int dtype) { return dtype == OSDN_BF16 ? 2 : 4; }
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
  bool valid() const { return lo != 0 && hi > lo; }
};
Range rng(const void* p, size_t bytes) {
  return Range{(uintptr_t)p, (uintptr_t)p + bytes};
}
bool overlap(Range a, Range b) {
  return a.valid() && b.valid() && a.lo < b.hi && b.lo < a.hi;
}
bool same(Range a, Range b) { return a.lo == b.lo && a.hi == b.hi; }

// Outputs must not overlap inputs or each other, except for the exact
// in-place pairs listed in `allowed` (output index, input index).
template <int NO, int NI>
bool aliasing_ok(const Range (&outs)[NO], const Range (&ins)[NI],
                 const int (*allowed)[2], int nallowed) {
  for (int i = 0; i < NO; ++i) {
    for (int j = 0; j < NI; ++j) {
      if (!overlap(outs[i], ins[j])) continue;
      bool ok = false;
      for (int a = 0; a < nallowed; ++a)
        if (allowed[a][0] == i && allowed[a][1] == j && same(outs[i], ins[j]))
          ok = true;
      if (!ok) return false;
    }
    for (int j = i + 1; j < NO; ++j)
      if (overlap(outs[i], outs[j])) return false;
  }
  return true;
}

// The gated forward forms K~ inside the engine at chunk 64 where that layout
// fits; otherwise it goes through the preconditioned keys in the workspace.
bool gated_fused(int Dk, int Dv, int chunk, int dtype) {
  return chunk == osdn::kPrecondChunk &&
         osdn::gated_fused_supported(Dk, Dv, dtype == OSDN_BF16);
}

// Workspace layout of a two-phase forward (osdn_forward, osdn_gated_forward).
// Fused (phase 2 forms K~ itself from the phase-1 records): the phase-1
// scratch at 0, the phase-2 scratch right after it, both live at once.
// Otherwise: K~ at 0, then one region shared by the two phases. The size
// queries return `total` and the launch paths take their offsets from the
// same struct, so the two cannot disagree.
struct Layout {
  bool fused;
  size_t kt_off, p1_off, p2_off, total;
};

Layout two_phase_layout(int B, int H, int T, int Dk, int dtype, bool fused,
                        size_t p1, size_t p2) {
  Layout l{};
  l.fused = fused;
  if (fused) {
    l.kt_off = 0;
    l.p1_off = 0;
    l.p2_off = p1;
    l.total = p1 + p2;
  } else {
    const size_t kt = round256((size_t)B * H * T * Dk * elem(dtype));
    l.kt_off = 0;
    l.p1_off = l.p2_off = kt;
    l.total = kt + (p1 > p2 ? p1 : p2);
  }
  return l;
}

}  // namespace

extern "C" {

const char* osdn_strerror(int status) {
  switch (status) {
    case OSDN_OK: return "ok";
    case OSDN_ERR_NULL_ARG: return "a required pointer argument is NULL";
    case OSDN_ERR_BAD_DIMS: return "bad dimensions: B, H and T must be >= 0";
    case OSDN_ERR_UNSUPPORTED:
      return "unsupported combination of Dk, Dv, chunk and dtype";
    case OSDN_ERR_WORKSPACE: return "workspace missing or too small";
    case OSDN_ERR_ALIASING:
      return "an output overlaps an input or another output";
    case OSDN_ERR_HIP: return "the HIP runtime rejected a kernel launch";
  }
  return "unknown status";
}

int osdn_forward_supported(int Dk, int Dv, int chunk, int dtype) {
  if (!dim_ok(Dk) || !dim_ok(Dv) || !chunk_ok(chunk)) return 0;
  if (dtype != OSDN_F32 && dtype != OSDN_BF16) return 0;
  return osdn::osdn_chunk_supported(Dk, Dv, chunk, dtype == OSDN_BF16) ? 1 : 0;
}

size_t osdn_precond_workspace_bytes(int B, int H, int T, int Dk, int dtype) {
  if (B < 0 || H < 0 || T < 0 || !dim_ok(Dk) ||
      (dtype != OSDN_F32 && dtype != OSDN_BF16))
    return 0;
  return round256(osdn::precond_workspace_bytes(B, H, T, Dk, dtype == OSDN_BF16));
}

static size_t chunk_ws_bytes(int B, int H, int T, int Dk, int Dv, int chunk,
                             int dtype, int gdn2) {
  if (B < 0 || H < 0 || T < 0 || !dim_ok(Dk) || !dim_ok(Dv) ||
      !chunk_ok(chunk) || (dtype != OSDN_F32 && dtype != OSDN_BF16))
    return 0;
  return round256(osdn::wy_workspace_bytes(B, H, T, Dk, Dv, chunk,
                                           dtype == OSDN_BF16, gdn2));
}

size_t osdn_chunk_workspace_bytes(int B, int H, int T, int Dk, int Dv,
                                  int chunk, int dtype) {
  if (!osdn_forward_supported(Dk, Dv, chunk, dtype)) return 0;
  return chunk_ws_bytes(B, H, T, Dk, Dv, chunk, dtype, 0);
}

size_t gdn2_forward_workspace_bytes(int B, int H, int T, int Dk, int Dv,
                                    int chunk, int dtype) {
  if (!gdn2_forward_supported(Dk, Dv, chunk, dtype)) return 0;
  return chunk_ws_bytes(B, H, T, Dk, Dv, chunk, dtype, 1);
}

static Layout osdn_layout(int B, int H, int T, int Dk, int Dv, int chunk,
                          int dtype) {
  // chunk = 64: phase 2 forms K~ itself from the phase-1 records
  return two_phase_layout(
      B, H, T, Dk, dtype, chunk == osdn::kPrecondChunk,
      osdn_precond_workspace_bytes(B, H, T, Dk, dtype),
      osdn_chunk_workspace_bytes(B, H, T, Dk, Dv, chunk, dtype));
}

size_t osdn_forward_workspace_bytes(int B, int H, int T, int Dk, int Dv,
                                    int chunk, int dtype) {
  if (B < 0 || H < 0 || T < 0 || !osdn_forward_supported(Dk, Dv, chunk, dtype))
    return 0;
  return osdn_layout(B, H, T, Dk, Dv, chunk, dtype).total;
}

int osdn_precond_scan(int B, int H, int T, int Dk, int dtype, const void* k,
                      const float* beta, const float* r, float eta,
                      const float* d0, void* ktilde, float* d_T, float* rho,
                      float* q_geo, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (B < 0 || H < 0 || T < 0) return OSDN_ERR_BAD_DIMS;
  // Pointers of zero-size tensors may be NULL.
  if ((size_t)B * H * T > 0 && (!k || !beta)) return OSDN_ERR_NULL_ARG;
  if (!dim_ok(Dk) || (dtype != OSDN_F32 && dtype != OSDN_BF16))
    return OSDN_ERR_UNSUPPORTED;
  const size_t need = osdn_precond_workspace_bytes(B, H, T, Dk, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need ||
                   ((uintptr_t)workspace & 255) != 0))
    return OSDN_ERR_WORKSPACE;
  if ((size_t)B * H == 0) return OSDN_OK;
  const size_t BH = (size_t)B * H, es = elem(dtype);
  const Range ins[] = {rng(k, BH * T * Dk * es), rng(beta, BH * T * 4),
                       rng(r, r ? BH * T * 4 : 0), rng(d0, d0 ? BH * Dk * 4 : 0)};
  const Range outs[] = {rng(ktilde, ktilde ? BH * T * Dk * es : 0),
                        rng(d_T, d_T ? BH * Dk * 4 : 0), rng(workspace, need),
                        rng(rho, rho ? BH * T * 4 : 0),
                        rng(q_geo, q_geo ? BH * 4 : 0)};
  const int allowed[][2] = {{1, 3}};  // d_T == d0
  if (!aliasing_ok(outs, ins, allowed, 1)) return OSDN_ERR_ALIASING;
  osdn::PrecondArgs a{B, H, T, Dk, dtype == OSDN_BF16, k, beta, r, eta, d0,
                      ktilde, d_T, workspace, rho, q_geo};
  const int rc = osdn::launch_precond_scan(a, (hipStream_t)stream);
  if (rc == -1) return OSDN_ERR_UNSUPPORTED;
  return rc == 0 ? OSDN_OK : OSDN_ERR_HIP;
}

int osdn_forward(int B, int H, int T, int Dk, int Dv, int chunk, int dtype,
                 const void* q, const void* k, const void* v,
                 const float* beta, const float* r, float eta,
                 const float* d0, const float* S0, float scale, void* o,
                 float* S_T, float* d_T, float* rho, float* q_geo,
                 void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || H < 0 || T < 0) return OSDN_ERR_BAD_DIMS;
  if ((size_t)B * H * T > 0 && (!q || !k || !v || !beta || !o))
    return OSDN_ERR_NULL_ARG;
  if (!osdn_forward_supported(Dk, Dv, chunk, dtype)) return OSDN_ERR_UNSUPPORTED;
  const size_t need = osdn_forward_workspace_bytes(B, H, T, Dk, Dv, chunk, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need ||
                   ((uintptr_t)workspace & 255) != 0))
    return OSDN_ERR_WORKSPACE;
  if ((size_t)B * H == 0) return OSDN_OK;

  const size_t BH = (size_t)B * H, es = elem(dtype);
  const Range ins[] = {rng(q, BH * T * Dk * es), rng(k, BH * T * Dk * es),
                       rng(v, BH * T * Dv * es), rng(beta, BH * T * 4),
                       rng(r, r ? BH * T * 4 : 0), rng(d0, d0 ? BH * Dk * 4 : 0),
                       rng(S0, S0 ? BH * Dv * Dk * 4 : 0)};
  const Range outs[] = {rng(o, BH * T * Dv * es),
                        rng(S_T, S_T ? BH * Dv * Dk * 4 : 0),
                        rng(d_T, d_T ? BH * Dk * 4 : 0),
                        rng(workspace, need), rng(rho, rho ? BH * T * 4 : 0),
                        rng(q_geo, q_geo ? BH * 4 : 0)};
  const int allowed[][2] = {{1, 6}, {2, 5}};  // S_T == S0, d_T == d0
  if (!aliasing_ok(outs, ins, allowed, 2)) return OSDN_ERR_ALIASING;

  hipStream_t s = (hipStream_t)stream;
  unsigned char* wsb = static_cast<unsigned char*>(workspace);
  const Layout lay = osdn_layout(B, H, T, Dk, Dv, chunk, dtype);
  int rc;
  if (lay.fused) {
    // phase-1 scratch (records, then entry values of d), then the phase-2
    // operands; K~ is formed inside phase 2
    osdn::PrecondArgs pa{B, H, T, Dk, dtype == OSDN_BF16, k, beta, r, eta, d0,
                         nullptr, d_T, wsb + lay.p1_off, rho, q_geo};
    rc = osdn::launch_precond_scan(pa, s);
    if (rc == -1) return OSDN_ERR_UNSUPPORTED;
    if (rc != 0) return OSDN_ERR_HIP;
    const int nch = (T + chunk - 1) / chunk;
    const float* prec = reinterpret_cast<const float*>(wsb + lay.p1_off);
    const float* pdent = prec + BH * (size_t)nch * osdn::kRecStride;
    osdn::ChunkArgs ca{B, H, T, Dk, Dv, chunk, dtype == OSDN_BF16, q, k,
                       nullptr, v, beta, S0, scale, o, S_T,
                       nullptr, nullptr, nullptr, wsb + lay.p2_off, prec, pdent};
    rc = osdn::launch_osdn_fused(ca, s);
  } else {
    // workspace: the preconditioned keys, then scratch shared by the phases
    void* kt = wsb + lay.kt_off;
    osdn::PrecondArgs pa{B, H, T, Dk, dtype == OSDN_BF16, k, beta, r, eta, d0,
                         kt, d_T, wsb + lay.p1_off, rho, q_geo};
    rc = osdn::launch_precond_scan(pa, s);
    if (rc == -1) return OSDN_ERR_UNSUPPORTED;
    if (rc != 0) return OSDN_ERR_HIP;
    osdn::ChunkArgs ca{B, H, T, Dk, Dv, chunk, dtype == OSDN_BF16, q, k,
                       kt, v, beta, S0, scale, o, S_T,
                       nullptr, nullptr, nullptr, wsb + lay.p2_off};
    rc = osdn::launch_osdn_chunk(ca, s);
  }
  if (rc == -1) return OSDN_ERR_UNSUPPORTED;
  return rc == 0 ? OSDN_OK : OSDN_ERR_HIP;
}

int osdn_chunk_forward(int B, int H, int T, int Dk, int Dv, int chunk,
                       int dtype, const void* q, const void* k,
                       const void* ktilde, const void* v, const float* beta,
                       const float* S0, float scale, void* o, float* S_T,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || H < 0 || T < 0) return OSDN_ERR_BAD_DIMS;
  if ((size_t)B * H * T > 0 && (!q || !k || !ktilde || !v || !beta || !o))
    return OSDN_ERR_NULL_ARG;
  if (!osdn_forward_supported(Dk, Dv, chunk, dtype)) return OSDN_ERR_UNSUPPORTED;
  const size_t need = osdn_chunk_workspace_bytes(B, H, T, Dk, Dv, chunk, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need ||
                   ((uintptr_t)workspace & 255) != 0))
    return OSDN_ERR_WORKSPACE;
  if ((size_t)B * H == 0) return OSDN_OK;
  const size_t BH = (size_t)B * H, es = elem(dtype);
  const Range ins[] = {rng(q, BH * T * Dk * es), rng(k, BH * T * Dk * es),
                       rng(ktilde, BH * T * Dk * es), rng(v, BH * T * Dv * es),
                       rng(beta, BH * T * 4), rng(S0, S0 ? BH * Dv * Dk * 4 : 0)};
  const Range outs[] = {rng(o, BH * T * Dv * es),
                        rng(S_T, S_T ? BH * Dv * Dk * 4 : 0),
                        rng(workspace, need)};
  const int allowed[][2] = {{1, 5}};  // S_T == S0
  if (!aliasing_ok(outs, ins, allowed, 1)) return OSDN_ERR_ALIASING;
  osdn::ChunkArgs ca{B, H, T, Dk, Dv, chunk, dtype == OSDN_BF16, q, k,
                     ktilde, v, beta, S0, scale, o, S_T,
                     nullptr, nullptr, nullptr, workspace};
  const int rc = osdn::launch_osdn_chunk(ca, (hipStream_t)stream);
  if (rc == -1) return OSDN_ERR_UNSUPPORTED;
  return rc == 0 ? OSDN_OK : OSDN_ERR_HIP;
}

int gdn2_forward_supported(int Dk, int Dv, int chunk, int dtype) {
  if (!dim_ok(Dk) || !dim_ok(Dv) || !chunk_ok(chunk)) return 0;
  if (dtype != OSDN_F32 && dtype != OSDN_BF16) return 0;
  return osdn::gdn2_chunk_supported(Dk, Dv, chunk, dtype == OSDN_BF16) ? 1 : 0;
}

int gdn2_forward(int B, int H, int T, int Dk, int Dv, int chunk, int dtype,
                 const void* q, const void* k, const void* v,
                 const float* log_alpha, const void* b, const void* w,
                 const float* S0, float scale, void* o, float* S_T,
                 void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || H < 0 || T < 0) return OSDN_ERR_BAD_DIMS;
  if ((size_t)B * H * T > 0 && (!q || !k || !v || !log_alpha || !b || !w || !o))
    return OSDN_ERR_NULL_ARG;
  if (!gdn2_forward_supported(Dk, Dv, chunk, dtype)) return OSDN_ERR_UNSUPPORTED;
  const size_t need = gdn2_forward_workspace_bytes(B, H, T, Dk, Dv, chunk, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need ||
                   ((uintptr_t)workspace & 255) != 0))
    return OSDN_ERR_WORKSPACE;
  if ((size_t)B * H == 0) return OSDN_OK;
  const size_t BH = (size_t)B * H, es = elem(dtype);
  const Range ins[] = {rng(q, BH * T * Dk * es), rng(k, BH * T * Dk * es),
                       rng(v, BH * T * Dv * es), rng(log_alpha, BH * T * Dk * 4),
                       rng(b, BH * T * Dk * es), rng(w, BH * T * Dv * es),
                       rng(S0, S0 ? BH * Dv * Dk * 4 : 0)};
  const Range outs[] = {rng(o, BH * T * Dv * es),
                        rng(S_T, S_T ? BH * Dv * Dk * 4 : 0),
                        rng(workspace, need)};
  const int allowed[][2] = {{1, 6}};  // S_T == S0
  if (!aliasing_ok(outs, ins, allowed, 1)) return OSDN_ERR_ALIASING;
  osdn::ChunkArgs ca{B, H, T, Dk, Dv, chunk, dtype == OSDN_BF16, q, k,
                     nullptr, v, nullptr, S0, scale, o, S_T, log_alpha, b, w,
                     workspace};
  const int rc = osdn::launch_gdn2_chunk(ca, (hipStream_t)stream);
  if (rc == -1) return OSDN_ERR_UNSUPPORTED;
  return rc == 0 ? OSDN_OK : OSDN_ERR_HIP;
}

int osdn_decode(int B, int H, int T, int Dk, int Dv, int dtype, const void* q,
                const void* k, const void* v, const float* beta,
                const float* r, float eta, const float* log_alpha, float* S,
                float* d, float scale, void* o, void* stream) {
  if (B < 0 || H < 0 || T < 0) return OSDN_ERR_BAD_DIMS;
  const size_t BH = (size_t)B * H;
  if (BH * T > 0 && (!q || !k || !v || !beta || !S || !d || !o))
    return OSDN_ERR_NULL_ARG;
  if (!dim_ok(Dk) || !dim_ok(Dv) || (dtype != OSDN_F32 && dtype != OSDN_BF16))
    return OSDN_ERR_UNSUPPORTED;
  if (BH * T == 0) return OSDN_OK;
  const size_t es = elem(dtype);
  const Range ins[] = {rng(q, BH * T * Dk * es), rng(k, BH * T * Dk * es),
                       rng(v, BH * T * Dv * es), rng(beta, BH * T * 4),
                       rng(r, r ? BH * T * 4 : 0),
                       rng(log_alpha, log_alpha ? BH * T * Dk * 4 : 0)};
  const Range outs[] = {rng(o, BH * T * Dv * es), rng(S, BH * Dv * Dk * 4),
                        rng(d, BH * Dk * 4)};
  if (!aliasing_ok(outs, ins, nullptr, 0)) return OSDN_ERR_ALIASING;
  osdn::DecodeArgs a{B, H, T, Dk, Dv, dtype == OSDN_BF16, 0, q, k, v, beta, r,
                     eta, log_alpha, nullptr, nullptr, S, d, scale, o};
  const int rc = osdn::launch_decode(a, (hipStream_t)stream);
  if (rc == -1) return OSDN_ERR_UNSUPPORTED;
  return rc == 0 ? OSDN_OK : OSDN_ERR_HIP;
}

int gdn2_decode(int B, int H, int T, int Dk, int Dv, int dtype, const void* q,
                const void* k, const void* v, const float* log_alpha,
                const void* b, const void* w, float* S, float scale, void* o,
                void* stream) {
  if (B < 0 || H < 0 || T < 0) return OSDN_ERR_BAD_DIMS;
  const size_t BH = (size_t)B * H;
  if (BH * T > 0 && (!q || !k || !v || !log_alpha || !b || !w || !S || !o))
    return OSDN_ERR_NULL_ARG;
  if (!dim_ok(Dk) || !dim_ok(Dv) || (dtype != OSDN_F32 && dtype != OSDN_BF16))
    return OSDN_ERR_UNSUPPORTED;
  if (BH * T == 0) return OSDN_OK;
  const size_t es = elem(dtype);
  const Range ins[] = {rng(q, BH * T * Dk * es), rng(k, BH * T * Dk * es),
                       rng(v, BH * T * Dv * es), rng(log_alpha, BH * T * Dk * 4),
                       rng(b, BH * T * Dk * es), rng(w, BH * T * Dv * es)};
  const Range outs[] = {rng(o, BH * T * Dv * es), rng(S, BH * Dk * Dv * 4)};
  if (!aliasing_ok(outs, ins, nullptr, 0)) return OSDN_ERR_ALIASING;
  osdn::DecodeArgs a{B, H, T, Dk, Dv, dtype == OSDN_BF16, 1, q, k, v, nullptr,
                     nullptr, 0.f, log_alpha, b, w, S, nullptr, scale, o};
  const int rc = osdn::launch_decode(a, (hipStream_t)stream);
  if (rc == -1) return OSDN_ERR_UNSUPPORTED;
  return rc == 0 ? OSDN_OK : OSDN_ERR_HIP;
}

size_t osdn_backward_workspace_bytes(int B, int H, int T, int Dk, int Dv) {
  if (B < 0 || H < 0 || T < 0 || !dim_ok(Dk) || !dim_ok(Dv)) return 0;
  return osdn::backward_workspace_bytes(B, H, T, Dk, Dv);
}

int osdn_backward(int B, int H, int T, int Dk, int Dv, int dtype,
                  const void* q, const void* k, const void* v,
                  const float* beta, const float* r, float eta,
                  const float* d0, const float* S0, float scale,
                  const void* dout, const float* dS_T, const float* dd_T,
                  float* dq, float* dk, float* dv, float* dbeta, float* dr,
                  float* deta, float* dd0, float* dS0, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (B < 0 || H < 0 || T < 0) return OSDN_ERR_BAD_DIMS;
  const size_t BH = (size_t)B * H;
  if (BH > 0 && (!deta || !dd0 || !dS0)) return OSDN_ERR_NULL_ARG;
  if (BH * T > 0 && (!q || !k || !v || !beta || !dout || !dq || !dk || !dv ||
                     !dbeta || !dr))
    return OSDN_ERR_NULL_ARG;
  if (!dim_ok(Dk) || !dim_ok(Dv) || (dtype != OSDN_F32 && dtype != OSDN_BF16))
    return OSDN_ERR_UNSUPPORTED;
  const size_t need = osdn_backward_workspace_bytes(B, H, T, Dk, Dv);
  if (need > 0 && (!workspace || workspace_bytes < need ||
                   ((uintptr_t)workspace & 255) != 0))
    return OSDN_ERR_WORKSPACE;
  if (BH == 0) return OSDN_OK;
  const size_t es = elem(dtype);
  const Range ins[] = {rng(q, BH * T * Dk * es), rng(k, BH * T * Dk * es),
                       rng(v, BH * T * Dv * es), rng(beta, BH * T * 4),
                       rng(r, r ? BH * T * 4 : 0), rng(d0, d0 ? BH * Dk * 4 : 0),
                       rng(S0, S0 ? BH * Dv * Dk * 4 : 0),
                       rng(dout, BH * T * Dv * es),
                       rng(dS_T, dS_T ? BH * Dv * Dk * 4 : 0),
                       rng(dd_T, dd_T ? BH * Dk * 4 : 0)};
  const Range outs[] = {rng(dq, BH * T * Dk * 4), rng(dk, BH * T * Dk * 4),
                        rng(dv, BH * T * Dv * 4), rng(dbeta, BH * T * 4),
                        rng(dr, BH * T * 4), rng(deta, BH * 4),
                        rng(dd0, BH * Dk * 4), rng(dS0, BH * Dv * Dk * 4),
                        rng(workspace, need)};
  if (!aliasing_ok(outs, ins, nullptr, 0)) return OSDN_ERR_ALIASING;
  osdn::BackwardArgs a{B, H, T, Dk, Dv, dtype == OSDN_BF16, q, k, v, beta, r,
                       eta, d0, S0, scale, dout, dS_T, dd_T, dq, dk, dv, dbeta,
                       dr, deta, dd0, dS0, workspace};
  const int rc = osdn::launch_backward(a, (hipStream_t)stream);
  if (rc == -1) return OSDN_ERR_UNSUPPORTED;
  return rc == 0 ? OSDN_OK : OSDN_ERR_HIP;
}

size_t osdn_gated_backward_workspace_bytes(int B, int H, int T, int Dk, int Dv) {
  if (B < 0 || H < 0 || T < 0 || !dim_ok(Dk) || !dim_ok(Dv)) return 0;
  return osdn::gated_backward_workspace_bytes(B, H, T, Dk, Dv, 0);
}

int osdn_gated_backward(int B, int H, int T, int Dk, int Dv, int dtype,
                        const void* q, const void* k, const void* v,
                        const float* beta, const float* r, float eta,
                        const float* log_alpha, const float* d0,
                        const float* S0, float scale, const void* dout,
                        const float* dS_T, const float* dd_T, float* dq,
                        float* dk, float* dv, float* dbeta, float* dr,
                        float* deta, float* dlog_alpha, float* dd0,
                        float* dS0, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (B < 0 || H < 0 || T < 0) return OSDN_ERR_BAD_DIMS;
  const size_t BH = (size_t)B * H;
  if (BH > 0 && (!deta || !dd0 || !dS0)) return OSDN_ERR_NULL_ARG;
  if (BH * T > 0 && (!q || !k || !v || !beta || !log_alpha || !dout || !dq ||
                     !dk || !dv || !dbeta || !dr || !dlog_alpha))
    return OSDN_ERR_NULL_ARG;
  if (!dim_ok(Dk) || !dim_ok(Dv) || (dtype != OSDN_F32 && dtype != OSDN_BF16))
    return OSDN_ERR_UNSUPPORTED;
  const size_t need = osdn_gated_backward_workspace_bytes(B, H, T, Dk, Dv);
  if (need > 0 && (!workspace || workspace_bytes < need ||
                   ((uintptr_t)workspace & 255) != 0))
    return OSDN_ERR_WORKSPACE;
  if (BH == 0) return OSDN_OK;
  const size_t es = elem(dtype);
  const Range ins[] = {rng(q, BH * T * Dk * es), rng(k, BH * T * Dk * es),
                       rng(v, BH * T * Dv * es), rng(beta, BH * T * 4),
                       rng(r, r ? BH * T * 4 : 0), rng(log_alpha, BH * T * Dk * 4),
                       rng(d0, d0 ? BH * Dk * 4 : 0),
                       rng(S0, S0 ? BH * Dv * Dk * 4 : 0),
                       rng(dout, BH * T * Dv * es),
                       rng(dS_T, dS_T ? BH * Dv * Dk * 4 : 0),
                       rng(dd_T, dd_T ? BH * Dk * 4 : 0)};
  const Range outs[] = {rng(dq, BH * T * Dk * 4), rng(dk, BH * T * Dk * 4),
                        rng(dv, BH * T * Dv * 4), rng(dbeta, BH * T * 4),
                        rng(dr, BH * T * 4), rng(deta, BH * 4),
                        rng(dlog_alpha, BH * T * Dk * 4),
                        rng(dd0, BH * Dk * 4), rng(dS0, BH * Dv * Dk * 4),
                        rng(workspace, need)};
  if (!aliasing_ok(outs, ins, nullptr, 0)) return OSDN_ERR_ALIASING;
  osdn::GatedBackwardArgs a{};
  a.B = B; a.H = H; a.T = T; a.Dk = Dk; a.Dv = Dv;
  a.bf16 = dtype == OSDN_BF16; a.gdn2 = 0;
  a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha;
  a.beta = beta; a.r = r; a.eta = eta; a.d0 = d0; a.S0 = S0; a.scale = scale;
  a.dout = dout; a.dST = dS_T; a.ddT = dd_T;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dla = dlog_alpha;
  a.dbeta = dbeta; a.dr = dr; a.deta = deta; a.dd0 = dd0; a.dS0 = dS0;
  a.ws = workspace;
  const int rc = osdn::launch_gated_backward(a, (hipStream_t)stream);
  if (rc == -1) return OSDN_ERR_UNSUPPORTED;
  return rc == 0 ? OSDN_OK : OSDN_ERR_HIP;
}

size_t gdn2_backward_workspace_bytes(int B, int H, int T, int Dk, int Dv) {
  if (B < 0 || H < 0 || T < 0 || !dim_ok(Dk) || !dim_ok(Dv)) return 0;
  return osdn::gated_backward_workspace_bytes(B, H, T, Dk, Dv, 1);
}

int gdn2_backward(int B, int H, int T, int Dk, int Dv, int dtype,
                  const void* q, const void* k, const void* v,
                  const float* log_alpha, const void* b, const void* w,
                  const float* S0, float scale, const void* dout,
                  const float* dS_T, float* dq, float* dk, float* dv,
                  float* dlog_alpha, float* db, float* dw, float* dS0,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || H < 0 || T < 0) return OSDN_ERR_BAD_DIMS;
  const size_t BH = (size_t)B * H;
  if (BH > 0 && !dS0) return OSDN_ERR_NULL_ARG;
  if (BH * T > 0 && (!q || !k || !v || !log_alpha || !b || !w || !dout ||
                     !dq || !dk || !dv || !dlog_alpha || !db || !dw))
    return OSDN_ERR_NULL_ARG;
  if (!dim_ok(Dk) || !dim_ok(Dv) || (dtype != OSDN_F32 && dtype != OSDN_BF16))
    return OSDN_ERR_UNSUPPORTED;
  const size_t need = gdn2_backward_workspace_bytes(B, H, T, Dk, Dv);
  if (need > 0 && (!workspace || workspace_bytes < need ||
                   ((uintptr_t)workspace & 255) != 0))
    return OSDN_ERR_WORKSPACE;
  if (BH == 0) return OSDN_OK;
  const size_t es = elem(dtype);
  const Range ins[] = {rng(q, BH * T * Dk * es), rng(k, BH * T * Dk * es),
                       rng(v, BH * T * Dv * es), rng(log_alpha, BH * T * Dk * 4),
                       rng(b, BH * T * Dk * es), rng(w, BH * T * Dv * es),
                       rng(S0, S0 ? BH * Dk * Dv * 4 : 0),
                       rng(dout, BH * T * Dv * es),
                       rng(dS_T, dS_T ? BH * Dk * Dv * 4 : 0)};
  const Range outs[] = {rng(dq, BH * T * Dk * 4), rng(dk, BH * T * Dk * 4),
                        rng(dv, BH * T * Dv * 4),
                        rng(dlog_alpha, BH * T * Dk * 4),
                        rng(db, BH * T * Dk * 4), rng(dw, BH * T * Dv * 4),
                        rng(dS0, BH * Dk * Dv * 4), rng(workspace, need)};
  if (!aliasing_ok(outs, ins, nullptr, 0)) return OSDN_ERR_ALIASING;
  osdn::GatedBackwardArgs a{};
  a.B = B; a.H = H; a.T = T; a.Dk = Dk; a.Dv = Dv;
  a.bf16 = dtype == OSDN_BF16; a.gdn2 = 1;
  a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.b = b; a.w = w;
  a.S0 = S0; a.scale = scale; a.dout = dout; a.dST = dS_T;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dla = dlog_alpha; a.db = db; a.dw = dw;
  a.dS0 = dS0; a.ws = workspace;
  const int rc = osdn::launch_gated_backward(a, (hipStream_t)stream);
  if (rc == -1) return OSDN_ERR_UNSUPPORTED;
  return rc == 0 ? OSDN_OK : OSDN_ERR_HIP;
}

int osdn_gated_forward_supported(int Dk, int Dv, int chunk, int dtype) {
  return gdn2_forward_supported(Dk, Dv, chunk, dtype);
}

static Layout gated_layout(int B, int H, int T, int Dk, int Dv, int chunk,
                           int dtype) {
  // chunk = 64 where that engine layout fits: the engine forms K~ from the
  // phase-1 records
  return two_phase_layout(B, H, T, Dk, dtype,
                          gated_fused(Dk, Dv, chunk, dtype),
                          osdn_precond_workspace_bytes(B, H, T, Dk, dtype),
                          chunk_ws_bytes(B, H, T, Dk, Dv, chunk, dtype, 1));
}

size_t osdn_gated_forward_workspace_bytes(int B, int H, int T, int Dk, int Dv,
                                          int chunk, int dtype) {
  if (B < 0 || H < 0 || T < 0 ||
      !osdn_gated_forward_supported(Dk, Dv, chunk, dtype))
    return 0;
  return gated_layout(B, H, T, Dk, Dv, chunk, dtype).total;
}

int osdn_gated_forward(int B, int H, int T, int Dk, int Dv, int chunk,
                       int dtype, const void* q, const void* k, const void* v,
                       const float* beta, const float* r, float eta,
                       const float* log_alpha, const float* d0,
                       const float* S0, float scale, void* o, float* S_T,
                       float* d_T, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (B < 0 || H < 0 || T < 0) return OSDN_ERR_BAD_DIMS;
  if ((size_t)B * H * T > 0 && (!q || !k || !v || !beta || !log_alpha || !o))
    return OSDN_ERR_NULL_ARG;
  if (!osdn_gated_forward_supported(Dk, Dv, chunk, dtype))
    return OSDN_ERR_UNSUPPORTED;
  const size_t need =
      osdn_gated_forward_workspace_bytes(B, H, T, Dk, Dv, chunk, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need ||
                   ((uintptr_t)workspace & 255) != 0))
    return OSDN_ERR_WORKSPACE;
  if ((size_t)B * H == 0) return OSDN_OK;
  const size_t BH = (size_t)B * H, es = elem(dtype);
  const Range ins[] = {rng(q, BH * T * Dk * es), rng(k, BH * T * Dk * es),
                       rng(v, BH * T * Dv * es), rng(beta, BH * T * 4),
                       rng(r, r ? BH * T * 4 : 0), rng(log_alpha, BH * T * Dk * 4),
                       rng(d0, d0 ? BH * Dk * 4 : 0),
                       rng(S0, S0 ? BH * Dv * Dk * 4 : 0)};
  const Range outs[] = {rng(o, BH * T * Dv * es),
                        rng(S_T, S_T ? BH * Dv * Dk * 4 : 0),
                        rng(d_T, d_T ? BH * Dk * 4 : 0),
                        rng(workspace, need)};
  const int allowed[][2] = {{1, 7}, {2, 6}};  // S_T == S0, d_T == d0
  if (!aliasing_ok(outs, ins, allowed, 2)) return OSDN_ERR_ALIASING;
  hipStream_t s = (hipStream_t)stream;
  unsigned char* wsb = static_cast<unsigned char*>(workspace);
  const Layout lay = gated_layout(B, H, T, Dk, Dv, chunk, dtype);
  int rc;
  if (lay.fused) {
    // phase-1 records and entry values of d, then the engine's operands
    osdn::PrecondArgs pa{B, H, T, Dk, dtype == OSDN_BF16, k, beta, r, eta, d0,
                         nullptr, d_T, wsb + lay.p1_off, nullptr, nullptr};
    rc = osdn::launch_precond_scan(pa, s);
    if (rc == -1) return OSDN_ERR_UNSUPPORTED;
    if (rc != 0) return OSDN_ERR_HIP;
    const int nch = (T + chunk - 1) / chunk;
    const float* prec = reinterpret_cast<const float*>(wsb + lay.p1_off);
    const float* pdent = prec + BH * (size_t)nch * osdn::kRecStride;
    osdn::ChunkArgs ca{B, H, T, Dk, Dv, chunk, dtype == OSDN_BF16, q, k,
                       nullptr, v, beta, S0, scale, o, S_T,
                       log_alpha, nullptr, nullptr, wsb + lay.p2_off, prec, pdent};
    rc = osdn::launch_osdn_gated_fused(ca, s);
  } else {
    void* kt = wsb + lay.kt_off;
    osdn::PrecondArgs pa{B, H, T, Dk, dtype == OSDN_BF16, k, beta, r, eta, d0,
                         kt, d_T, wsb + lay.p1_off, nullptr, nullptr};
    rc = osdn::launch_precond_scan(pa, s);
    if (rc == -1) return OSDN_ERR_UNSUPPORTED;
    if (rc != 0) return OSDN_ERR_HIP;
    osdn::ChunkArgs ca{B, H, T, Dk, Dv, chunk, dtype == OSDN_BF16, q, k,
                       kt, v, beta, S0, scale, o, S_T,
                       log_alpha, nullptr, nullptr, wsb + lay.p2_off};
    rc = osdn::launch_osdn_gated_chunk(ca, s);
  }
  if (rc == -1) return OSDN_ERR_UNSUPPORTED;
  return rc == 0 ? OSDN_OK : OSDN_ERR_HIP;
}

}  // extern "C"
