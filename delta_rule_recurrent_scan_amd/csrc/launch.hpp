// Host-side argument bundles passed from the C-ABI layer to the kernel
// launchers. Pointers are device pointers owned by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace osdn {

// Phase-1 chunk length and the layout of its per-chunk fp32 record
// {lp_0..lp_C (lp_t = log of the gate product before token t), 3 pad,
// g (C step sizes), V (C x C), c_t = P_C / P_{t+1} (C gate ratios), P_C,
// 3 pad}; the entry values of d follow all records. Every field starts on a
// 16-byte boundary.
constexpr int kPrecondChunk = 64;
constexpr int kRecLp = 0, kRecG = kPrecondChunk + 4, kRecV = 2 * kPrecondChunk + 4;
constexpr int kRecCf = kRecV + kPrecondChunk * kPrecondChunk;
constexpr int kRecPc = kRecCf + kPrecondChunk;
constexpr int kRecStride = kRecPc + 4;
static_assert(kRecV % 4 == 0 && kRecCf % 4 == 0 && kRecStride % 4 == 0,
              "record fields on 16-byte boundaries");

struct PrecondArgs {
  int B, H, T, Dk;
  int bf16;                 // 1: k and ktilde are bf16, 0: fp32
  const void* k;            // [B,H,T,Dk]
  const float* beta;        // [B,H,T]
  const float* r;           // [B,H,T] or null (gate off)
  float eta;
  const float* d0;          // [B,H,Dk] or null (ones)
  void* ktilde;             // [B,H,T,Dk] in the k dtype, or null
  float* dT;                // [B,H,Dk] or null
  void* ws;                 // precond_workspace_bytes(...) bytes, 16-byte aligned
  float* rho;               // [B,H,T] residual contraction ratios, or null
  float* qgeo;              // [B,H] their geometric mean, or null
};

// Arguments of the chunked WY engine. OSDN uses ktilde and beta, with the
// state stored [B,H,Dv,Dk]; GDN-2 uses log_alpha, b and w, with the state
// stored [B,H,Dk,Dv].
struct ChunkArgs {
  int B, H, T, Dk, Dv, chunk;
  int bf16;
  const void* q;            // [B,H,T,Dk]
  const void* k;            // [B,H,T,Dk]
  const void* ktilde;       // OSDN: [B,H,T,Dk]
  const void* v;            // [B,H,T,Dv]
  const float* beta;        // OSDN: [B,H,T]
  const float* S0;          // or null (zeros)
  float scale;
  void* o;                  // [B,H,T,Dv]
  float* ST;                // or null
  const float* log_alpha;   // GDN-2: [B,H,T,Dk] fp32
  const void* b;            // GDN-2: [B,H,T,Dk] erase gate
  const void* w;            // GDN-2: [B,H,T,Dv] write gate
  void* ws;                 // wy_workspace_bytes(...) bytes, 16-byte aligned
  // OSDN with K~ formed inside the engine (chunk == kPrecondChunk): the
  // phase-1 records and entry values of d (ktilde unused).
  const float* prec;
  const float* pdent;
};

// Arguments of the recurrent decode kernels: T tokens through the token
// recurrence with the state updated in place. OSDN: beta, r, eta, d; state
// [B,H,Dv,Dk]. GDN-2: log_alpha, b, w; state [B,H,Dk,Dv].
struct DecodeArgs {
  int B, H, T, Dk, Dv;
  int bf16;
  int gdn2;
  const void* q;            // [B,H,T,Dk]
  const void* k;            // [B,H,T,Dk]
  const void* v;            // [B,H,T,Dv]
  const float* beta;        // OSDN: [B,H,T]
  const float* r;           // OSDN: [B,H,T] or null
  float eta;
  const float* log_alpha;   // [B,H,T,Dk] (OSDN: null = no decay)
  const void* b;            // GDN-2: [B,H,T,Dk]
  const void* w;            // GDN-2: [B,H,T,Dv]
  float* S;                 // in/out
  float* d;                 // OSDN: [B,H,Dk] in/out
  float scale;
  void* o;                  // [B,H,T,Dv]
};

// Arguments of the OSDN backward (the adjoint of the token recurrence):
// inputs as in the forward plus the output adjoints; gradients fp32 in the
// inputs' layouts, eta's per (batch, head).
struct BackwardArgs {
  int B, H, T, Dk, Dv;
  int bf16;
  const void* q;            // [B,H,T,Dk]
  const void* k;            // [B,H,T,Dk]
  const void* v;            // [B,H,T,Dv]
  const float* beta;        // [B,H,T]
  const float* r;           // [B,H,T] or null (ones)
  float eta;
  const float* d0;          // [B,H,Dk] or null (ones)
  const float* S0;          // [B,H,Dv,Dk] or null (zeros)
  float scale;
  const void* dout;         // [B,H,T,Dv], dtype of q
  const float* dST;         // [B,H,Dv,Dk] or null (zeros)
  const float* ddT;         // [B,H,Dk] or null (zeros)
  float *dq, *dk, *dv;      // [B,H,T,Dk], [B,H,T,Dk], [B,H,T,Dv]
  float *dbeta, *dr;        // [B,H,T]
  float* deta;              // [B,H]
  float *dd0, *dS0;         // [B,H,Dk], [B,H,Dv,Dk]
  void* ws;                 // backward_workspace_bytes
};

// Arguments of the gate-aware backward (GDN-2, or OSDN on a per-channel-
// decay backbone): the forward's inputs plus the output adjoints; gradients
// fp32 in the inputs' layouts. OSDN: beta, r, eta, d0 and their gradients,
// state [B,H,Dv,Dk]; GDN-2: b, w and theirs, state [B,H,Dk,Dv].
struct GatedBackwardArgs {
  int B, H, T, Dk, Dv;
  int bf16;
  int gdn2;
  const void *q, *k, *v;    // [B,H,T,Dk], [B,H,T,Dk], [B,H,T,Dv]
  const float* log_alpha;   // [B,H,T,Dk]
  const void *b, *w;        // GDN-2: [B,H,T,Dk], [B,H,T,Dv]
  const float *beta, *r;    // OSDN: [B,H,T] (r null: ones)
  float eta;
  const float *d0, *S0;     // OSDN d0 [B,H,Dk] or null; S0 or null
  float scale;
  const void* dout;         // [B,H,T,Dv], dtype of q
  const float *dST, *ddT;   // or null (zeros); ddT OSDN only
  float *dq, *dk, *dv, *dla;
  float *db, *dw;           // GDN-2
  float *dbeta, *dr, *deta, *dd0;  // OSDN
  float* dS0;
  void* ws;                 // gated_backward_workspace_bytes
};

// Each returns a hipError_t-compatible code (0 = success) or -1 when the
// (dims, dtype) combination has no kernel instance.
int launch_precond_scan(const PrecondArgs& a, hipStream_t s);
// Device scratch of the chunk-parallel phase 1: per chunk, the record
// {log gate prefix, g, V} and the entry value of d.
size_t precond_workspace_bytes(int B, int H, int T, int Dk, int bf16);
int launch_osdn_chunk(const ChunkArgs& a, hipStream_t s);
int launch_osdn_fused(const ChunkArgs& a, hipStream_t s);
// OSDN on a per-channel-decay backbone: ktilde, beta and log_alpha used,
// state [B,H,Dv,Dk]; workspace as for GDN-2 (wy_workspace_bytes(..., 1)).
int launch_osdn_gated_chunk(const ChunkArgs& a, hipStream_t s);
// The same forming K~ inside the engine from prec / pdent (chunk ==
// kPrecondChunk); workspace: the phase-1 scratch stays live beside it.
int launch_osdn_gated_fused(const ChunkArgs& a, hipStream_t s);
// Whether the fused gated variant has an instance for (Dk, Dv, dtype) at
// chunk kPrecondChunk (its LDS layout fits).
bool gated_fused_supported(int Dk, int Dv, int bf16);
int launch_gdn2_chunk(const ChunkArgs& a, hipStream_t s);
int launch_decode(const DecodeArgs& a, hipStream_t s);
// Device scratch of the backward: per token the residual u_t and the
// preconditioner d_t, and the state every 64 tokens and after the last.
size_t backward_workspace_bytes(int B, int H, int T, int Dk, int Dv);
int launch_backward(const BackwardArgs& a, hipStream_t s);
// Device scratch of the gate-aware backward: per token the preconditioner
// (OSDN only), the state every 64 tokens and after the last, and one
// 64-token interval of states per stream.
size_t gated_backward_workspace_bytes(int B, int H, int T, int Dk, int Dv, int gdn2);
int launch_gated_backward(const GatedBackwardArgs& a, hipStream_t s);
bool osdn_chunk_supported(int Dk, int Dv, int chunk, int bf16);
bool gdn2_chunk_supported(int Dk, int Dv, int chunk, int bf16);
// Device scratch of the chunk engine: per chunk, the S0-independent operands
// of the chunk step (GDN-2 has two more: its decayed queries and decays).
size_t wy_workspace_bytes(int B, int H, int T, int Dk, int Dv, int chunk,
                          int bf16, int gdn2);

// Kernel timing hooks (no-ops unless enabled through osdn_kernel_timing):
// an event on stream s before the kernel `name` is launched and one after.
// ktimer_before returns the handle of the record it started (-1 when timing
// is off or no event was available); ktimer_after completes that record only.
int ktimer_before(hipStream_t s, const char* name);
void ktimer_after(hipStream_t s, int handle);

}  // namespace osdn
