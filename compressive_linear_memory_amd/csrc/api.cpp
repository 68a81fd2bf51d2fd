// libinfini C ABI: validation, workspace layout and launch order.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <initializer_list>
#include <mutex>

#include "../../include/infini.h"
#include "kernels.h"

namespace {

using infini::Geometry;

constexpr int kMaxChunkSegments = INFINI_CHUNK_SEGMENTS;   // segments whose snapshots live in the workspace at once

bool valid_problem(const infini_problem_t* p, infini_status_t* why) {
  if (!p) { *why = INFINI_ERR_NULL; return false; }
  // batch = 0 or seq_len = 0 is an empty problem: nothing to compute, the
  // state passes through
  if (p->batch < 0 || p->q_heads <= 0 || p->kv_heads <= 0 || p->seq_len < 0 ||
      p->head_dim <= 0 || p->seg_len <= 0) { *why = INFINI_ERR_SHAPE; return false; }
  if (p->q_heads % p->kv_heads != 0) { *why = INFINI_ERR_SHAPE; return false; }
  if (p->head_dim != 32 && p->head_dim != 64 && p->head_dim != 128) {
    *why = INFINI_ERR_UNSUPPORTED; return false;
  }
  if (p->dtype != INFINI_FP32 && p->dtype != INFINI_BF16) { *why = INFINI_ERR_UNSUPPORTED; return false; }
  if (p->feature_map != INFINI_FEATURE_ELU1 && p->feature_map != INFINI_FEATURE_TAYLOR2) {
    *why = INFINI_ERR_UNSUPPORTED; return false;
  }
  // Every index the kernels form must fit comfortably in 64 bits and every
  // per-call count in 32 bits.
  const double elems = (double)p->batch * p->q_heads * p->seq_len * p->head_dim;
  if (elems > 9.0e15 || (double)p->batch * p->q_heads > 2147483647.0) { *why = INFINI_ERR_SHAPE; return false; }
  return true;
}

Geometry geometry(const infini_problem_t* p) {
  Geometry g;
  g.B = p->batch; g.Hq = p->q_heads; g.Hkv = p->kv_heads; g.N = p->seq_len;
  g.D = p->head_dim; g.L = p->seg_len; g.dtype = p->dtype; g.fmap = p->feature_map;
  // the last segment may be shorter; formed in 64 bits (seq_len + seg_len
  // can exceed the 32-bit range)
  g.S = (int)(((int64_t)p->seq_len + p->seg_len - 1) / p->seg_len);
  return g;
}

int chunk_segments(const Geometry& g) {
  int c = kMaxChunkSegments;
  if (const char* e = getenv("INFINI_CHUNK_SEGMENTS")) {   // test hook: force multi-chunk paths
    const int v = atoi(e);
    if (v >= 1 && v < c) c = v;
  }
  return g.S < c ? g.S : c;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

size_t elem_bytes(const Geometry& g) { return g.dtype == INFINI_FP32 ? 4 : 2; }

// ---- workspace layouts (byte offsets, 256-aligned)

struct FwdWs { size_t Msnap, zsnap, MsnapT, dz, Amem, total; };

// Features per key of the problem's memory path (the rows of M).
size_t feature_dim(const Geometry& g) { return g.fmap == INFINI_FEATURE_TAYLOR2 ? infini::taylor_dim(g.D) : g.D; }

// Only the forward entry points take the Taylor feature map.
bool elu_only(const infini_problem_t* p) { return p && p->feature_map != INFINI_FEATURE_ELU1; }
// parts: key splits per segment of the matrix-core memory phase (0: the
// library's choice for g)
FwdWs fwd_layout(const Geometry& g, int parts_of = 0) {
  const size_t C = (size_t)(g.S < kMaxChunkSegments ? g.S : kMaxChunkSegments);
  const size_t bk = (size_t)g.B * g.Hkv;
  FwdWs w{};
  size_t off = 0;
  if (g.fmap == INFINI_FEATURE_TAYLOR2) {   // fp32 snapshots over D' features, and the retrieved rows
    const size_t nf = feature_dim(g);
    w.Msnap = off; off = align_up(off + bk * C * nf * g.D * 4);
    w.zsnap = off; off = align_up(off + bk * C * nf * 4);
    w.Amem = off;  off = align_up(off + (size_t)g.B * g.Hq * C * g.L * g.D * 4);
    w.MsnapT = w.dz = off;
    w.total = off;
    // the matrix-core path needs only the starting state's retrieval terms
    if (infini::taylor_mfma_supported(g)) w.total = std::max(w.total, infini::taylor_mfma_m0_bytes(g));
    return w;
  }
  // The matrix-core path keeps its per-segment dM parts (one per key split)
  // where the generic path keeps fp32 snapshots.
  const bool mfma = infini::fwd_mfma_supported(g);
  const size_t parts = mfma ? (size_t)(parts_of > 0 ? parts_of : infini::delta_splits(g)) : 1;
  w.Msnap = off; off = align_up(off + bk * C * parts * g.D * g.D * 4);
  w.zsnap = off; off = align_up(off + bk * C * g.D * 4);
  w.MsnapT = off; off = align_up(off + (mfma ? bk * C * g.D * g.D * 2 : 0));
  w.dz = off;     off = align_up(off + (mfma ? bk * C * parts * g.D * 4 : 0));
  w.Amem = off;
  w.total = off;
  return w;
}

// Memory phase + attention phase over segments [s0, s1), kernel family by problem.
hipError_t run_fwd_chunk(const Geometry& g, const FwdWs& lay, char* base, const void* Q,
                         const void* K, const void* V, const float* beta, const float* Min,
                         const float* zin, void* O, float* M_S, float* z_S, float* lse, int s0,
                         int s1, hipStream_t st, bool memory, bool attend) {
  float* Msnap = reinterpret_cast<float*>(base + lay.Msnap);
  float* zsnap = reinterpret_cast<float*>(base + lay.zsnap);
  if (g.fmap == INFINI_FEATURE_TAYLOR2) {
    float* Amem = reinterpret_cast<float*>(base + lay.Amem);
    if (memory) {
      hipError_t e = infini::launch_taylor_sweep(g, K, V, Min, zin, M_S, z_S, Msnap, zsnap, s0, s1, st);
      if (e != hipSuccess) return e;
    }
    if (!attend) return hipSuccess;
    hipError_t e = infini::launch_taylor_retrieve(g, Q, Msnap, zsnap, Amem, s0, s1, st);
    if (e != hipSuccess) return e;
    return infini::launch_fwd_generic(g, Q, K, V, beta, nullptr, nullptr, O, lse, s0, s1, st, Amem);
  }
  const bool mfma = infini::fwd_mfma_supported(g);
  void* MsnapT = mfma ? base + lay.MsnapT : nullptr;
  if (memory) {
    // The matrix-core path keeps per-segment dM in the fp32 snapshot area
    // (it reads only the bf16 transposed snapshots).
    hipError_t e = mfma ? infini::launch_sweep_mfma(g, K, V, Min, zin, M_S, z_S, Msnap,
                                                    reinterpret_cast<float*>(base + lay.dz), MsnapT,
                                                    zsnap, s0, s1, st)
                        : infini::launch_sweep(g, K, V, Min, zin, M_S, z_S, Msnap, zsnap, s0, s1, st);
    if (e != hipSuccess) return e;
  }
  if (attend) {
    if (mfma) return infini::launch_fwd_mfma(g, Q, K, V, beta, MsnapT, zsnap, O, lse, s0, s1, st);
    return infini::launch_fwd_generic(g, Q, K, V, beta, Msnap, zsnap, O, lse, s0, s1, st);
  }
  return hipSuccess;
}

struct BwdWs { size_t Mst, zst, Msnap, zsnap, dMc, dzc, dMsnap, dzsnap, lse, Dd, dden, dnum, dbp, dbacc, dbs, dlt, dltz, total; };
BwdWs bwd_layout(const Geometry& g) {
  if (infini::bwd_short_supported(g)) {   // the fused backward needs only its dbeta partials
    BwdWs w{};
    w.dbs = 0;
    w.total = align_up((size_t)g.B * g.Hq * 4);
    return w;
  }
  const size_t C = (size_t)(g.S < kMaxChunkSegments ? g.S : kMaxChunkSegments);
  const size_t bk = (size_t)g.B * g.Hkv;
  const size_t rows = (size_t)g.B * g.Hq * C * g.L;
  const size_t D = g.D;
  BwdWs w;
  size_t off = 0;
  w.Mst = off;    off = align_up(off + bk * D * D * 4);
  w.zst = off;    off = align_up(off + bk * D * 4);
  w.Msnap = off;  off = align_up(off + bk * C * D * D * 4);
  w.zsnap = off;  off = align_up(off + bk * C * D * 4);
  w.dMc = off;    off = align_up(off + bk * D * D * 4);
  w.dzc = off;    off = align_up(off + bk * D * 4);
  w.dMsnap = off; off = align_up(off + bk * C * D * D * 4);
  w.dzsnap = off; off = align_up(off + bk * C * D * 4);
  w.lse = off;    off = align_up(off + rows * 4);
  w.Dd = off;     off = align_up(off + rows * 4);
  w.dden = off;   off = align_up(off + rows * 4);
  w.dnum = off;   off = align_up(off + rows * D * 4);
  w.dbp = off;    off = align_up(off + (size_t)g.B * g.Hq * C * infini::bwd_q_row_blocks(g) * 4);
  w.dbacc = off;  off = align_up(off + (size_t)g.Hq * 4);
  w.dbs = off;    off = align_up(off + (size_t)g.B * g.Hq * 4);
  // matrix-core path: per-segment scratch of the memory phase (its deltas,
  // key-split parts included), reused by the reverse scan for the segments'
  // retrieval terms; Msnap then holds the bf16 transposed snapshots and their
  // bf16 remainders (the same bytes as one fp32 copy)
  w.dlt = w.dltz = 0;
  if (infini::bwd_long_mfma_supported(g)) {
    const size_t ns = (size_t)infini::delta_splits(g);
    w.dlt = off;  off = align_up(off + bk * C * ns * D * D * 4);
    w.dltz = off; off = align_up(off + bk * C * ns * D * 4);
  }
  w.total = off;
  return w;
}

// ---- aliasing

struct Span { const void* p; size_t n; };
bool overlap(Span a, Span b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}
bool any_overlap(const Span* outs, int no, const Span* ins, int ni) {
  for (int i = 0; i < no; ++i) {
    for (int j = 0; j < ni; ++j) if (overlap(outs[i], ins[j])) return true;
    for (int j = i + 1; j < no; ++j) if (overlap(outs[i], outs[j])) return true;
  }
  return false;
}

// The kernels move tensors in 16-byte vectors: every tensor pointer but
// beta, dbeta and lse must be 16-byte aligned (NULL counts as aligned).
bool misaligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (reinterpret_cast<uintptr_t>(p) & 15) return true;
  return false;
}

infini_status_t hip_status(hipError_t e) { return e == hipSuccess ? INFINI_OK : INFINI_ERR_HIP; }

#define TRY(expr)                                       \
  do {                                                  \
    hipError_t e_ = (expr);                             \
    if (e_ != hipSuccess) return hip_status(e_);        \
  } while (0)

// ---- static scratch of the allocation-free decode
//
// One array per device, in device memory, for the whole process.  In host
// code its name stands for a host-side handle, not a device address: the
// address is taken once per device with hipGetSymbolAddress and only that
// pointer is passed to kernels.
__device__ __align__(256) unsigned char scratch[INFINI_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (set up on its first use).
hipError_t scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* infini_status_string(infini_status_t s) {
  // a C caller may pass any int; read the bits rather than the enum value
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case INFINI_OK: return "ok";
    case INFINI_ERR_NULL: return "a required pointer is NULL";
    case INFINI_ERR_SHAPE: return "invalid shape (batch, seq_len >= 0, other dims > 0, q_heads % kv_heads == 0, sizes within limits)";
    case INFINI_ERR_UNSUPPORTED: return "unsupported head_dim (32, 64, 128), dtype, or a tensor pointer not 16-byte aligned";
    case INFINI_ERR_ALIAS: return "an output buffer overlaps an input or another output";
    case INFINI_ERR_WORKSPACE: return "workspace is NULL or too small";
    case INFINI_ERR_HIP: return "HIP launch or runtime error";
    case INFINI_ERR_SCRATCH: return "the problem needs more scratch than the allocation-free entry point's static maximum (INFINI_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

int infini_version(void) { return INFINI_VERSION; }

const char* infini_fwd_path(const infini_problem_t* p) {
  infini_status_t why;
  if (!valid_problem(p, &why)) return nullptr;
  const Geometry g = geometry(p);
  if (g.fmap == INFINI_FEATURE_TAYLOR2)
    return infini::taylor_mfma_supported(g) ? "mfma_bf16_taylor2" : "generic_fp32_taylor2";
  if (infini::fwd_short_supported(g)) return "mfma_bf16_short";
  return infini::fwd_mfma_supported(g) ? "mfma_bf16" : "generic_fp32";
}

size_t infini_fwd_workspace_bytes(const infini_problem_t* p) {
  infini_status_t why;
  if (!valid_problem(p, &why)) return 0;
  return fwd_layout(geometry(p)).total;
}

size_t infini_fwd_saved_bytes(const infini_problem_t* p) {
  infini_status_t why;
  if (!valid_problem(p, &why)) return 0;
  return (size_t)p->batch * p->q_heads * p->seq_len * 4;
}

size_t infini_bwd_workspace_bytes(const infini_problem_t* p) {
  infini_status_t why;
  if (!valid_problem(p, &why) || elu_only(p)) return 0;
  return bwd_layout(geometry(p)).total;
}

// lens: device int32 [batch] of sequence lengths (variable-length batch), or
// NULL when every sequence has p->seq_len tokens.
static infini_status_t attn_fwd_impl(const infini_problem_t* p, const int32_t* lens, const void* Q,
                                     const void* K, const void* V, const float* beta, const float* M0,
                                     const float* z0, void* O, float* M_S, float* z_S, float* lse, void* ws,
                                     size_t ws_bytes, void* stream) {
  infini_status_t why;
  if (!valid_problem(p, &why)) return why;
  Geometry g = geometry(p);
  g.lens = lens;
  if (reinterpret_cast<uintptr_t>(lens) & 3) return INFINI_ERR_UNSUPPORTED;
  const size_t eb = elem_bytes(g);
  const size_t nq = (size_t)g.B * g.Hq * g.N * g.D, nkv = (size_t)g.B * g.Hkv * g.N * g.D;
  const size_t nf = feature_dim(g);
  const size_t nM = (size_t)g.B * g.Hkv * nf * g.D * 4, nz = (size_t)g.B * g.Hkv * nf * 4;
  // tensors of no elements may be null (torch gives them no storage)
  if ((nq && (!Q || !O)) || (nkv && (!K || !V)) || !beta || (nM && (!M_S || !z_S))) return INFINI_ERR_NULL;
  if ((M0 == nullptr) != (z0 == nullptr)) return INFINI_ERR_NULL;
  if (misaligned({Q, K, V, M0, z0, O, M_S, z_S, ws})) return INFINI_ERR_UNSUPPORTED;
  const FwdWs lay = fwd_layout(g);
  // the fused short-segment kernel keeps its state on chip and needs none;
  // the matrix-core Taylor forward (empty starting memory) forms no states
  const bool taylor_fast = infini::taylor_mfma_supported(g);
  const size_t need = infini::fwd_short_supported(g) ? 0
                      : taylor_fast                  ? (M0 ? infini::taylor_mfma_m0_bytes(g) : 0)
                                                     : lay.total;
  if ((need && !ws) || ws_bytes < need) return INFINI_ERR_WORKSPACE;
  const Span outs[] = {{O, nq * eb}, {M_S, nM}, {z_S, nz}, {lse, lse ? (size_t)g.B * g.Hq * g.N * 4 : 0},
                       {ws, need}};
  const Span ins[] = {{Q, nq * eb}, {K, nkv * eb}, {V, nkv * eb}, {beta, (size_t)g.Hq * 4},
                      {M0, M0 ? nM : 0}, {z0, z0 ? nz : 0}, {lens, lens ? (size_t)g.B * 4 : 0}};
  if (any_overlap(outs, 5, ins, 7)) return INFINI_ERR_ALIAS;

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (g.N == 0) {                         // no tokens: the state passes through
    TRY(infini::launch_state_copy(M_S, M0, nM / 4, st));
    TRY(infini::launch_state_copy(z_S, z0, nz / 4, st));
    return INFINI_OK;
  }
  if (g.B == 0) return INFINI_OK;
  if (lens) {                             // rows past each sequence's end are zero
    TRY(infini::launch_zero_tail(O, lens, g.B, g.Hq, g.N, g.D * eb / 4, st));
    TRY(infini::launch_zero_tail(lse, lens, g.B, g.Hq, g.N, 1, st));
  }
  if (infini::fwd_short_supported(g)) {   // state stays on chip for the whole call
    TRY(infini::launch_fwd_short(g, Q, K, V, beta, M0, z0, O, M_S, z_S, lse, st));
    return INFINI_OK;
  }
  if (taylor_fast) {
    TRY(infini::launch_taylor_mfma(g, Q, K, V, beta, M0, z0, O, M_S, z_S, lse, ws, st));
    return INFINI_OK;
  }
  char* base = static_cast<char*>(ws);
  const int C = chunk_segments(g);
  for (int s0 = 0; s0 < g.S; s0 += C) {
    const int s1 = s0 + C < g.S ? s0 + C : g.S;
    const float* Min = s0 == 0 ? M0 : M_S;
    const float* zin = s0 == 0 ? z0 : z_S;
    TRY(run_fwd_chunk(g, lay, base, Q, K, V, beta, Min, zin, O, M_S, z_S, lse, s0, s1, st, true, true));
  }
  return INFINI_OK;
}

infini_status_t infini_attn_fwd(const infini_problem_t* p, const void* Q, const void* K,
                                const void* V, const float* beta, const float* M0, const float* z0,
                                void* O, float* M_S, float* z_S, float* lse, void* ws,
                                size_t ws_bytes, void* stream) {
  return attn_fwd_impl(p, nullptr, Q, K, V, beta, M0, z0, O, M_S, z_S, lse, ws, ws_bytes, stream);
}

infini_status_t infini_attn_fwd_varlen(const infini_problem_t* p, const int32_t* seq_lens, const void* Q,
                                       const void* K, const void* V, const float* beta, const float* M0,
                                       const float* z0, void* O, float* M_S, float* z_S, float* lse, void* ws,
                                       size_t ws_bytes, void* stream) {
  return attn_fwd_impl(p, seq_lens, Q, K, V, beta, M0, z0, O, M_S, z_S, lse, ws, ws_bytes, stream);
}

infini_status_t infini_fwd_memory(const infini_problem_t* p, const void* K, const void* V,
                                  const float* M0, const float* z0, float* M_S, float* z_S,
                                  void* ws, size_t ws_bytes, void* stream) {
  infini_status_t why;
  if (!valid_problem(p, &why)) return why;
  if (elu_only(p)) return INFINI_ERR_UNSUPPORTED;
  const Geometry g = geometry(p);
  const size_t eb = elem_bytes(g);
  const size_t nkv = (size_t)g.B * g.Hkv * g.N * g.D;
  const size_t nM = (size_t)g.B * g.Hkv * g.D * g.D * 4, nz = (size_t)g.B * g.Hkv * g.D * 4;
  if ((nkv && (!K || !V)) || (nM && (!M_S || !z_S))) return INFINI_ERR_NULL;
  if ((M0 == nullptr) != (z0 == nullptr)) return INFINI_ERR_NULL;
  if (misaligned({K, V, M0, z0, M_S, z_S, ws})) return INFINI_ERR_UNSUPPORTED;
  if (g.S > kMaxChunkSegments) return INFINI_ERR_SHAPE;
  const FwdWs lay = fwd_layout(g);
  if ((lay.total && !ws) || ws_bytes < lay.total) return INFINI_ERR_WORKSPACE;
  const Span outs[] = {{M_S, nM}, {z_S, nz}, {ws, lay.total}};
  const Span ins[] = {{K, nkv * eb}, {V, nkv * eb}, {M0, M0 ? nM : 0}, {z0, z0 ? nz : 0}};
  if (any_overlap(outs, 3, ins, 4)) return INFINI_ERR_ALIAS;
  if (g.N == 0 || g.B == 0) {  // no tokens: the state passes through
    TRY(infini::launch_state_copy(M_S, M0, nM / 4, static_cast<hipStream_t>(stream)));
    TRY(infini::launch_state_copy(z_S, z0, nz / 4, static_cast<hipStream_t>(stream)));
    return INFINI_OK;
  }
  TRY(run_fwd_chunk(g, lay, static_cast<char*>(ws), nullptr, K, V, nullptr, M0, z0, nullptr, M_S, z_S,
                    nullptr, 0, g.S, static_cast<hipStream_t>(stream), true, false));
  return INFINI_OK;
}

infini_status_t infini_fwd_attend(const infini_problem_t* p, const void* Q, const void* K,
                                  const void* V, const float* beta, void* O, float* lse,
                                  const void* ws, size_t ws_bytes, void* stream) {
  infini_status_t why;
  if (!valid_problem(p, &why)) return why;
  if (elu_only(p)) return INFINI_ERR_UNSUPPORTED;
  const Geometry g = geometry(p);
  const size_t eb = elem_bytes(g);
  const size_t nq = (size_t)g.B * g.Hq * g.N * g.D, nkv = (size_t)g.B * g.Hkv * g.N * g.D;
  if ((nq && (!Q || !O)) || (nkv && (!K || !V)) || !beta) return INFINI_ERR_NULL;
  if (misaligned({Q, K, V, O, ws})) return INFINI_ERR_UNSUPPORTED;
  if (g.S > kMaxChunkSegments) return INFINI_ERR_SHAPE;
  const FwdWs lay = fwd_layout(g);
  if ((lay.total && !ws) || ws_bytes < lay.total) return INFINI_ERR_WORKSPACE;
  const Span outs[] = {{O, nq * eb}, {lse, lse ? (size_t)g.B * g.Hq * g.N * 4 : 0}};
  const Span ins[] = {{Q, nq * eb}, {K, nkv * eb}, {V, nkv * eb}, {beta, (size_t)g.Hq * 4},
                      {ws, lay.total}};
  if (any_overlap(outs, 2, ins, 5)) return INFINI_ERR_ALIAS;
  if (g.N == 0 || g.B == 0) return INFINI_OK;
  TRY(run_fwd_chunk(g, lay, static_cast<char*>(const_cast<void*>(ws)), Q, K, V, beta, nullptr, nullptr, O,
                    nullptr, nullptr, lse, 0, g.S, static_cast<hipStream_t>(stream), false, true));
  return INFINI_OK;
}

static_assert(INFINI_STREAM_MAX_GROUP <= infini::kFwdMaxGroup, "a group's calls fit one call table");

namespace {
// Workspace of one pipeline stage of infini_fwd_stream: on the matrix-core
// path one forward workspace for a run of nc * S segments (nc <= group calls),
// else one per call.
size_t stream_stage_bytes(const Geometry& g, int group) {
  size_t b = (size_t)group * fwd_layout(g).total;
  if (infini::fwd_mfma_supported(g))
    for (int nc = 1; nc <= group; ++nc) {
      Geometry gg = g;
      gg.S = nc * g.S;
      b = std::max(b, fwd_layout(gg, infini::delta_splits(g)).total);
    }
  return b;
}
}  // namespace

size_t infini_fwd_stream_workspace_bytes(const infini_problem_t* p, int n_pipe, int group) {
  infini_status_t why;
  if (!valid_problem(p, &why) || elu_only(p) || n_pipe < 1 || group < 1 || group > INFINI_STREAM_MAX_GROUP) return 0;
  const Geometry g = geometry(p);
  if (g.S > kMaxChunkSegments) return 0;
  if (infini::fwd_mfma_supported(g) && group * g.S > kMaxChunkSegments) return 0;
  return (size_t)n_pipe * stream_stage_bytes(g, group);
}

infini_status_t infini_fwd_stream(const infini_problem_t* p, int n_launches, const void* const* Q,
                                  const void* const* K, const void* const* V, const float* beta,
                                  float* M, float* z, void* const* O, void* ws, size_t ws_bytes,
                                  int n_pipe, int group, void* mem_stream, void* const* att_streams,
                                  void* const* events) {
  infini_status_t why;
  if (!valid_problem(p, &why)) return why;
  if (elu_only(p)) return INFINI_ERR_UNSUPPORTED;
  if (n_launches < 1 || n_pipe < 1 || group < 1 || group > INFINI_STREAM_MAX_GROUP) return INFINI_ERR_SHAPE;
  if (p->seq_len == 0 || p->batch == 0) return INFINI_OK;  // no tokens: M and z stay as they are
  if (!Q || !K || !V || !O || !beta || !M || !z || !ws || !att_streams || !events) return INFINI_ERR_NULL;
  if (misaligned({M, z, ws})) return INFINI_ERR_UNSUPPORTED;
  const Geometry g = geometry(p);
  const bool mfma = infini::fwd_mfma_supported(g);
  if (g.S > kMaxChunkSegments || (mfma && group * g.S > kMaxChunkSegments)) return INFINI_ERR_SHAPE;
  const size_t stage = stream_stage_bytes(g, group);
  if (ws_bytes / (size_t)n_pipe < stage) return INFINI_ERR_WORKSPACE;
  for (int r = 0; r < n_pipe; ++r)
    if (!att_streams[r]) return INFINI_ERR_NULL;
  for (int r = 0; r < 2 * n_pipe; ++r)
    if (!events[r]) return INFINI_ERR_NULL;
  const size_t eb = elem_bytes(g);
  const size_t nq = (size_t)g.B * g.Hq * g.N * g.D, nkv = (size_t)g.B * g.Hkv * g.N * g.D;
  const size_t nM = (size_t)g.B * g.Hkv * g.D * g.D * 4, nz = (size_t)g.B * g.Hkv * g.D * 4;
  const size_t wsz = (size_t)n_pipe * stage;
  for (int i = 0; i < n_launches; ++i) {
    if (!Q[i] || !K[i] || !V[i] || !O[i]) return INFINI_ERR_NULL;
    if (misaligned({Q[i], K[i], V[i], O[i]})) return INFINI_ERR_UNSUPPORTED;
    const Span outs[] = {{O[i], nq * eb}, {M, nM}, {z, nz}, {ws, wsz}};
    const Span ins[] = {{Q[i], nq * eb}, {K[i], nkv * eb}, {V[i], nkv * eb}, {beta, (size_t)g.Hq * 4}};
    if (any_overlap(outs, 4, ins, 4)) return INFINI_ERR_ALIAS;
  }
  // Graph capture of this schedule is not supported: the streams are joined
  // by events that each group records again, and a capture of that pattern
  // has ended a process.  Refused before anything is issued.
  for (int r = -1; r < n_pipe; ++r) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    TRY(hipStreamIsCapturing(static_cast<hipStream_t>(r < 0 ? mem_stream : att_streams[r]), &cs));
    if (cs != hipStreamCaptureStatusNone) return INFINI_ERR_UNSUPPORTED;
  }
  const FwdWs lay = fwd_layout(g);
  hipStream_t sm = static_cast<hipStream_t>(mem_stream);
  char* base = static_cast<char*>(ws);
  // Group k (calls k*group ..) uses pipeline stage r = k % n_pipe: workspace
  // stage r, attention stream r, events r and n_pipe + r.
  for (int k = 0; k * group < n_launches; ++k) {
    const int r = k % n_pipe;
    const int i0 = k * group, nc = std::min(group, n_launches - i0);
    hipStream_t sa = static_cast<hipStream_t>(att_streams[r]);
    hipEvent_t ev_mem = static_cast<hipEvent_t>(events[r]);
    hipEvent_t ev_att = static_cast<hipEvent_t>(events[n_pipe + r]);
    char* w = base + (size_t)r * stage;
    // the stage's workspace is reused once the attention of group k - n_pipe is done
    if (k >= n_pipe) TRY(hipStreamWaitEvent(sm, ev_att, 0));
    if (mfma) {
      // one memory phase over the group's calls as one run of segments, then
      // one attention launch for all of them
      infini::FwdCallTable tab{};
      for (int j = 0; j < nc; ++j) {
        tab.Q[j] = static_cast<const __bf16*>(Q[i0 + j]);
        tab.K[j] = static_cast<const __bf16*>(K[i0 + j]);
        tab.V[j] = static_cast<const __bf16*>(V[i0 + j]);
        tab.O[j] = static_cast<__bf16*>(O[i0 + j]);
      }
      Geometry gg = g;
      gg.S = nc * g.S;
      const FwdWs lg = fwd_layout(gg, infini::delta_splits(g));
      TRY(infini::launch_sweep_mfma_group(g, tab, nc, M, z, M, z, reinterpret_cast<float*>(w + lg.Msnap),
                                          reinterpret_cast<float*>(w + lg.dz), w + lg.MsnapT,
                                          reinterpret_cast<float*>(w + lg.zsnap), sm));
      TRY(hipEventRecord(ev_mem, sm));
      TRY(hipStreamWaitEvent(sa, ev_mem, 0));
      TRY(infini::launch_fwd_mfma_group(g, tab, nc, beta, w + lg.MsnapT, reinterpret_cast<float*>(w + lg.zsnap),
                                        sa));
    } else {
      for (int j = 0; j < nc; ++j)
        TRY(run_fwd_chunk(g, lay, w + (size_t)j * lay.total, nullptr, K[i0 + j], V[i0 + j], nullptr, M, z,
                          nullptr, M, z, nullptr, 0, g.S, sm, true, false));
      TRY(hipEventRecord(ev_mem, sm));
      TRY(hipStreamWaitEvent(sa, ev_mem, 0));
      for (int j = 0; j < nc; ++j)
        TRY(run_fwd_chunk(g, lay, w + (size_t)j * lay.total, Q[i0 + j], K[i0 + j], V[i0 + j], beta, nullptr,
                          nullptr, O[i0 + j], nullptr, nullptr, nullptr, 0, g.S, sa, false, true));
    }
    TRY(hipEventRecord(ev_att, sa));
  }
  return INFINI_OK;
}

// Ms_in, zs_in: the forward's final state (both NULL: rebuilt from K, V, M0, z0).
static infini_status_t attn_bwd_impl(const infini_problem_t* p, const int32_t* lens, const void* Q,
                                     const void* K, const void* V, const float* beta, const float* M0,
                                     const float* z0, const float* Ms_in, const float* zs_in, const float* lse,
                                     const void* dO, const float* dM_S, const float* dz_S, void* dQ, void* dK,
                                     void* dV, float* dbeta, float* dM0, float* dz0, void* ws, size_t ws_bytes,
                                     void* stream) {
  infini_status_t why;
  if (!valid_problem(p, &why)) return why;
  if (elu_only(p)) return INFINI_ERR_UNSUPPORTED;
  Geometry g = geometry(p);
  g.lens = lens;
  if (reinterpret_cast<uintptr_t>(lens) & 3) return INFINI_ERR_UNSUPPORTED;
  const size_t eb = elem_bytes(g);
  const size_t nq = (size_t)g.B * g.Hq * g.N * g.D, nkv = (size_t)g.B * g.Hkv * g.N * g.D;
  const size_t nM = (size_t)g.B * g.Hkv * g.D * g.D * 4, nz = (size_t)g.B * g.Hkv * g.D * 4;
  // tensors of no elements may be null (torch gives them no storage)
  if ((nq && (!Q || !dO || !dQ)) || (nkv && (!K || !V || !dK || !dV)) || !beta || !dbeta) return INFINI_ERR_NULL;
  if ((M0 == nullptr) != (z0 == nullptr)) return INFINI_ERR_NULL;
  if ((Ms_in == nullptr) != (zs_in == nullptr)) return INFINI_ERR_NULL;
  if ((dM_S == nullptr) != (dz_S == nullptr)) return INFINI_ERR_NULL;
  if ((dM0 == nullptr) != (dz0 == nullptr)) return INFINI_ERR_NULL;
  if (misaligned({Q, K, V, M0, z0, Ms_in, zs_in, dO, dM_S, dz_S, dQ, dK, dV, dM0, dz0, ws}))
    return INFINI_ERR_UNSUPPORTED;
  const BwdWs lay = bwd_layout(g);
  if ((lay.total && !ws) || ws_bytes < lay.total) return INFINI_ERR_WORKSPACE;
  const Span outs[] = {{dQ, nq * eb}, {dK, nkv * eb}, {dV, nkv * eb}, {dbeta, (size_t)g.Hq * 4},
                       {dM0, dM0 ? nM : 0}, {dz0, dz0 ? nz : 0}, {ws, lay.total}};
  const Span ins[] = {{Q, nq * eb}, {K, nkv * eb}, {V, nkv * eb}, {beta, (size_t)g.Hq * 4},
                      {M0, M0 ? nM : 0}, {z0, z0 ? nz : 0}, {dO, nq * eb},
                      {dM_S, dM_S ? nM : 0}, {dz_S, dz_S ? nz : 0},
                      {lse, lse ? (size_t)g.B * g.Hq * g.N * 4 : 0}, {lens, lens ? (size_t)g.B * 4 : 0},
                      {Ms_in, Ms_in ? nM : 0}, {zs_in, zs_in ? nz : 0}};
  if (any_overlap(outs, 7, ins, 13)) return INFINI_ERR_ALIAS;

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (g.N == 0 || g.B == 0) {             // no tokens: the state's gradient passes through
    TRY(infini::launch_state_copy(dbeta, nullptr, (size_t)g.Hq, st));
    if (dM0) {
      TRY(infini::launch_state_copy(dM0, dM_S, nM / 4, st));
      TRY(infini::launch_state_copy(dz0, dz_S, nz / 4, st));
    }
    return INFINI_OK;
  }
  if (lens) {                             // rows past each sequence's end are zero
    TRY(infini::launch_zero_tail(dQ, lens, g.B, g.Hq, g.N, g.D * eb / 4, st));
    TRY(infini::launch_zero_tail(dK, lens, g.B, g.Hkv, g.N, g.D * eb / 4, st));
    TRY(infini::launch_zero_tail(dV, lens, g.B, g.Hkv, g.N, g.D * eb / 4, st));
  }
  char* base = static_cast<char*>(ws);
  auto F = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
  if (infini::bwd_short_supported(g)) {   // state and its gradient stay on chip
    TRY(infini::launch_bwd_short(g, Q, K, V, beta, M0, z0, dO, dM_S, dz_S, dQ, dK, dV, dbeta, dM0, dz0,
                                 F(lay.dbs), lse, st, Ms_in, zs_in));
    return INFINI_OK;
  }
  infini::BwdChunkWs w;
  w.lse = F(lay.lse); w.Dd = F(lay.Dd); w.dden = F(lay.dden); w.dnum = F(lay.dnum);
  w.dbeta_part = F(lay.dbp); w.dMsnap = F(lay.dMsnap); w.dzsnap = F(lay.dzsnap);
  float* Mst = F(lay.Mst); float* zst = F(lay.zst);
  float* Msnap = F(lay.Msnap); float* zsnap = F(lay.zsnap);
  float* dMc = F(lay.dMc); float* dzc = F(lay.dzc);
  float* dbacc = F(lay.dbacc);

  const int C = chunk_segments(g);
  const int nchunks = (g.S + C - 1) / C;
  const bool mf = infini::bwd_long_mfma_supported(g);
  // The chunks are walked last to first.  With more than one, the memory path
  // runs forward once to the state after the last chunk, and each chunk's
  // start state is then recovered by taking that chunk's updates away again
  // (linear in the number of chunks; the first chunk starts from M0 itself)
  // (or the forward's, when given).
  if (nchunks > 1) {
    if (Ms_in) {
      TRY(infini::launch_state_copy(Mst, Ms_in, nM / 4, st));
      TRY(infini::launch_state_copy(zst, zs_in, nz / 4, st));
    } else {
      TRY(infini::launch_sweep(g, K, V, M0, z0, Mst, zst, nullptr, nullptr, 0, g.S, st));
    }
  }
  for (int ci = nchunks - 1; ci >= 0; --ci) {
    const int s0 = ci * C;
    const int s1 = s0 + C < g.S ? s0 + C : g.S;
    const float* Mstart = M0;
    const float* zstart = z0;
    if (s0 > 0) {   // state at the chunk start
      TRY(infini::launch_sweep(g, K, V, Mst, zst, Mst, zst, nullptr, nullptr, s0, s1, st, nullptr, true));
      Mstart = Mst; zstart = zst;
    }
    if (mf) {   // snapshots as bf16 hi / lo pairs, transposed, from the matrix-core memory phase
      char* hi = base + lay.Msnap;
      char* lo = hi + (size_t)g.B * g.Hkv * (s1 - s0) * g.D * g.D * 2;
      TRY(infini::launch_sweep_mfma(g, K, V, Mstart, zstart, nullptr, nullptr, F(lay.dlt), F(lay.dltz), hi,
                                    zsnap, s0, s1, st, lo));
      TRY(infini::launch_bwd_q_mfma(g, Q, K, V, beta, hi, lo, zsnap, dO, dQ, w, lse, s0, s1, st));
    } else {
      TRY(infini::launch_sweep(g, K, V, Mstart, zstart, nullptr, nullptr, Msnap, zsnap, s0, s1, st));
      TRY(infini::launch_bwd_q(g, Q, K, V, beta, Msnap, zsnap, dO, dQ, w, lse, s0, s1, st));
    }
    const bool first = ci == nchunks - 1, last = ci == 0;
    TRY(infini::launch_dbeta_reduce(g, beta, w, dbacc, dbeta, s1 - s0, first, last, st));
    const float* dMin = first ? dM_S : dMc;
    const float* dzin = first ? dz_S : dzc;
    float* dMout = last ? dM0 : dMc;
    float* dzout = last ? dz0 : dzc;
    if (mf) TRY(infini::launch_rscan_mfma(g, Q, w, F(lay.dlt), F(lay.dltz), dMin, dzin, dMout, dzout, s0, s1, st));
    else TRY(infini::launch_rscan(g, Q, w, dMin, dzin, dMout, dzout, s0, s1, st));
    TRY(infini::launch_bwd_kv(g, Q, K, V, beta, dO, w, dK, dV, s0, s1, st));
  }
  return INFINI_OK;
}

infini_status_t infini_attn_bwd(const infini_problem_t* p, const void* Q, const void* K,
                                const void* V, const float* beta, const float* M0, const float* z0,
                                const float* lse, const void* dO, const float* dM_S,
                                const float* dz_S, void* dQ, void* dK, void* dV, float* dbeta,
                                float* dM0, float* dz0, void* ws, size_t ws_bytes, void* stream) {
  return attn_bwd_impl(p, nullptr, Q, K, V, beta, M0, z0, nullptr, nullptr, lse, dO, dM_S, dz_S, dQ, dK, dV, dbeta,
                       dM0, dz0, ws, ws_bytes, stream);
}

infini_status_t infini_attn_bwd_varlen(const infini_problem_t* p, const int32_t* seq_lens, const void* Q,
                                       const void* K, const void* V, const float* beta, const float* M0,
                                       const float* z0, const float* lse, const void* dO, const float* dM_S,
                                       const float* dz_S, void* dQ, void* dK, void* dV, float* dbeta,
                                       float* dM0, float* dz0, void* ws, size_t ws_bytes, void* stream) {
  return attn_bwd_impl(p, seq_lens, Q, K, V, beta, M0, z0, nullptr, nullptr, lse, dO, dM_S, dz_S, dQ, dK, dV, dbeta,
                       dM0, dz0, ws, ws_bytes, stream);
}

infini_status_t infini_attn_bwd_saved(const infini_problem_t* p, const int32_t* seq_lens, const void* Q,
                                      const void* K, const void* V, const float* beta, const float* M0,
                                      const float* z0, const float* M_S, const float* z_S, const float* lse,
                                      const void* dO, const float* dM_S, const float* dz_S, void* dQ, void* dK,
                                      void* dV, float* dbeta, float* dM0, float* dz0, void* ws, size_t ws_bytes,
                                      void* stream) {
  return attn_bwd_impl(p, seq_lens, Q, K, V, beta, M0, z0, M_S, z_S, lse, dO, dM_S, dz_S, dQ, dK, dV, dbeta, dM0,
                       dz0, ws, ws_bytes, stream);
}

// ---- streaming decode

// The geometry of one full segment of the decode problem (the shape of the
// caches and of the memory update that closes the segment).
static bool decode_problem(const infini_problem_t* p, int32_t pos, Geometry* seg, infini_status_t* why) {
  if (!valid_problem(p, why)) return false;
  if (elu_only(p)) { *why = INFINI_ERR_UNSUPPORTED; return false; }
  // a decode step carries at least one token of at least one sequence
  if (p->seq_len < 1 || p->batch < 1 || pos < 0 || (int64_t)pos + p->seq_len > p->seg_len) {
    *why = INFINI_ERR_SHAPE;
    return false;
  }
  infini_problem_t q = *p;
  q.seq_len = p->seg_len;
  *seg = geometry(&q);
  return true;
}

// The memory update that closes a segment and the key-split partials of the
// rows are never live together (same stream, one after the other), so they
// share the workspace.
static size_t decode_ws_bytes(const Geometry& seg, int Tn) {
  const size_t a = fwd_layout(seg).total, b = align_up(infini::decode_partial_bytes(seg, Tn));
  return a > b ? a : b;
}

size_t infini_decode_workspace_bytes(const infini_problem_t* p) {
  infini_status_t why;
  Geometry seg;
  if (!decode_problem(p, 0, &seg, &why)) return 0;
  return decode_ws_bytes(seg, p->seq_len);
}

// ws NULL with noalloc: the workspace is this device's static scratch.
static infini_status_t decode_impl(const infini_problem_t* p, int32_t pos, const void* Q, const void* K,
                                   const void* V, const float* beta, void* Kcache, void* Vcache,
                                   const float* M, const float* z, void* O, float* M_next, float* z_next,
                                   void* ws, size_t ws_bytes, void* stream, bool noalloc) {
  infini_status_t why;
  Geometry seg;
  if (!decode_problem(p, pos, &seg, &why)) return why;
  if (!Q || !K || !V || !beta || !Kcache || !Vcache || !O) return INFINI_ERR_NULL;
  if ((M == nullptr) != (z == nullptr)) return INFINI_ERR_NULL;
  const bool closes = pos + p->seq_len == p->seg_len;
  if (closes && (!M_next || !z_next)) return INFINI_ERR_NULL;
  if (misaligned({Q, K, V, Kcache, Vcache, M, z, O, M_next, z_next, ws})) return INFINI_ERR_UNSUPPORTED;
  const FwdWs lay = fwd_layout(seg);
  const size_t need = decode_ws_bytes(seg, p->seq_len);
  if (noalloc) {
    if (need > (size_t)INFINI_NOALLOC_SCRATCH_BYTES) return INFINI_ERR_SCRATCH;
  } else if (!ws || ws_bytes < need) {
    return INFINI_ERR_WORKSPACE;
  }
  const size_t eb = elem_bytes(seg);
  const size_t Tn = (size_t)p->seq_len;
  const size_t nq = (size_t)seg.B * seg.Hq * Tn * seg.D, nkv = (size_t)seg.B * seg.Hkv * Tn * seg.D;
  const size_t nc = (size_t)seg.B * seg.Hkv * seg.L * seg.D;
  const size_t nM = (size_t)seg.B * seg.Hkv * seg.D * seg.D * 4, nz = (size_t)seg.B * seg.Hkv * seg.D * 4;
  const Span outs[] = {{O, nq * eb}, {Kcache, nc * eb}, {Vcache, nc * eb},
                       {M_next, closes ? nM : 0}, {z_next, closes ? nz : 0}, {ws, noalloc ? 0 : need}};
  const Span ins[] = {{Q, nq * eb}, {K, nkv * eb}, {V, nkv * eb}, {beta, (size_t)seg.Hq * 4},
                      {M, M ? nM : 0}, {z, z ? nz : 0}};
  if (any_overlap(outs, 6, ins, 6)) return INFINI_ERR_ALIAS;
  if (noalloc) TRY(scratch_of_current_device(&ws));

  hipStream_t st = static_cast<hipStream_t>(stream);
  TRY(infini::launch_decode(seg, (int)Tn, pos, Q, K, V, beta, Kcache, Vcache, M, z, O,
                            static_cast<float*>(ws), st));
  if (closes)   // the segment is complete: fold it into the memory
    TRY(run_fwd_chunk(seg, lay, static_cast<char*>(ws), nullptr, Kcache, Vcache, nullptr, M, z, nullptr,
                      M_next, z_next, nullptr, 0, 1, st, true, false));
  return INFINI_OK;
}

infini_status_t infini_decode(const infini_problem_t* p, int32_t pos, const void* Q, const void* K,
                              const void* V, const float* beta, void* Kcache, void* Vcache,
                              const float* M, const float* z, void* O, float* M_next, float* z_next,
                              void* ws, size_t ws_bytes, void* stream) {
  return decode_impl(p, pos, Q, K, V, beta, Kcache, Vcache, M, z, O, M_next, z_next, ws, ws_bytes, stream,
                     false);
}

infini_status_t infini_decode_noalloc(const infini_problem_t* p, int32_t pos, const void* Q, const void* K,
                                      const void* V, const float* beta, void* Kcache, void* Vcache,
                                      const float* M, const float* z, void* O, float* M_next, float* z_next,
                                      void* stream) {
  return decode_impl(p, pos, Q, K, V, beta, Kcache, Vcache, M, z, O, M_next, z_next, nullptr, 0, stream, true);
}

}  // extern "C"
