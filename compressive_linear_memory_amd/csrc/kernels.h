// Host-side launch interface between api.cpp and the HIP kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace infini {

// One call's geometry, after validation.
struct Geometry {
  int B, Hq, Hkv, N, D, L, S;   // S = ceil(N / L) segments (of the longest sequence)
  int dtype;                    // 0 fp32, 1 bf16
  // Variable-length batch: device int32 [B], sequence b holds lens[b] <= N
  // tokens in the first rows of its N-row slot (clamped to [0, N] where
  // read).  NULL: every sequence has N tokens.
  const int* lens = nullptr;
  // Feature map of the memory path: 0 = ELU + 1 (feature dim D), 1 = the
  // second-order Taylor map (feature dim 1 + D + D^2).
  int fmap = 0;
  int G() const { return Hq / Hkv; }
};

// Second-order Taylor feature map (fp32 vector kernels, any dtype and head
// dim): the memory path over D' = taylor_dim(D) features, and the retrieval
// A_mem = phi(Q) M / (phi(Q) z + eps) of every row into Amem
// ([B][Hq][nseg * L][D] fp32, the layout the generic attention kernel reads).
// Msnap [B*Hkv][nseg][D'][D], zsnap [B*Hkv][nseg][D'].
size_t taylor_dim(int D);
hipError_t launch_taylor_sweep(const Geometry& g, const void* K, const void* V, const float* M_in,
                               const float* z_in, float* M_out, float* z_out, float* Msnap, float* zsnap,
                               int s_begin, int s_end, hipStream_t st);
hipError_t launch_taylor_retrieve(const Geometry& g, const void* Q, const float* Msnap, const float* zsnap,
                                  float* Amem, int s_begin, int s_end, hipStream_t st);

// Matrix-core Taylor forward (bf16, head_dim 64 or 128): the retrieval as
// polynomial-weighted attention over the earlier segments' keys (no
// per-segment state) plus, with a starting state, phi(q) M0 / phi(q) z0 per
// query; the local attention and gate; the final M_S ([B*Hkv][D'][D]) and
// z_S from K, V (and M0, z0).  m0ws: taylor_mfma_m0_bytes(g) bytes of
// scratch when M0 is given, else unused.
bool taylor_mfma_supported(const Geometry& g);
size_t taylor_mfma_m0_bytes(const Geometry& g);
hipError_t launch_taylor_mfma(const Geometry& g, const void* Q, const void* K, const void* V,
                              const float* beta, const float* M0, const float* z0, void* O, float* M_S, float* z_S,
                              float* lse, void* m0ws, hipStream_t st);

// Zero rows [lens[b], N) of every (b, h) slot of X ([B][H][N][row_words]
// 32-bit words per row): the rows past each sequence's end.
hipError_t launch_zero_tail(void* X, const int* lens, int B, int H, int N, size_t row_words, hipStream_t st);

// Memory path over segments [s_begin, s_end) of the call.
//   M_in/z_in: state before segment s_begin (NULL = empty memory).
//   M_out/z_out: state after segment s_end - 1 (NULL = not written; may equal M_in).
//   Msnap/zsnap: per-segment state before each segment, [B*Hkv][s_end-s_begin][D][D]
//   (NULL = not written).
//   MsnapT: optional bf16 copy of each snapshot, transposed ([c][a]), for the
//   matrix-core forward (NULL = not written).
//   subtract: take the segments' updates away instead (M_out = M_in -
//   sum sigma(K)^T V): walks back from a later state to an earlier one.
hipError_t launch_sweep(const Geometry& g, const void* K, const void* V,
                        const float* M_in, const float* z_in, float* M_out, float* z_out,
                        float* Msnap, float* zsnap, int s_begin, int s_end, hipStream_t st,
                        void* MsnapT = nullptr, bool subtract = false);

// bf16 matrix-core memory phase (head_dim 64 or 128): per-segment dM, dz into
// the scratch buffers dM [B*Hkv][nseg][D][D] and dz [B*Hkv][nseg][D], then the
// prefix over segments into MsnapT (bf16, transposed) and zsnap, and the state
// after the last segment into M_out / z_out (may equal M_in / z_in).
// Key splits per segment of the bf16 memory phase (dM and dz hold that many
// parts per segment).
int delta_splits(const Geometry& g);
// MsnapTlo, when given, receives bf16(M - bf16(M)) in the layout of MsnapT.
hipError_t launch_sweep_mfma(const Geometry& g, const void* K, const void* V, const float* M_in,
                             const float* z_in, float* M_out, float* z_out, float* dM, float* dz,
                             void* MsnapT, float* zsnap, int s_begin, int s_end, hipStream_t st,
                             void* MsnapTlo = nullptr);

// bf16 matrix-core forward (head_dim 64 or 128), reading MsnapT / zsnap.
bool fwd_mfma_supported(const Geometry& g);
hipError_t launch_fwd_mfma(const Geometry& g, const void* Q, const void* K, const void* V,
                           const float* beta, const void* MsnapT, const float* zsnap, void* O,
                           float* lse, int s_begin, int s_end, hipStream_t st);

// Several calls of the same shape (g: one call) in one memory-phase launch
// pair and one attention launch: call c's tensors in entry c.  The memory
// phase treats the calls' segments as one run of ncalls * g.S segments (the
// state carried through them in order), with delta_splits(g) parts per
// segment as each call alone would have, and publishes its states as
// launch_sweep_mfma does for that many segments; the attention launch reads
// them from there.
constexpr int kFwdMaxGroup = 8;
struct FwdCallTable {
  const __bf16* Q[kFwdMaxGroup];
  const __bf16* K[kFwdMaxGroup];
  const __bf16* V[kFwdMaxGroup];
  __bf16* O[kFwdMaxGroup];
};
hipError_t launch_sweep_mfma_group(const Geometry& g, const FwdCallTable& tab, int ncalls, const float* M_in,
                                   const float* z_in, float* M_out, float* z_out, float* dM, float* dz,
                                   void* MsnapT, float* zsnap, hipStream_t st);
hipError_t launch_fwd_mfma_group(const Geometry& g, const FwdCallTable& tab, int ncalls, const float* beta,
                                 const void* MsnapT, const float* zsnap, hipStream_t st);

// Fused short-segment forward (bf16, head_dim 64 or 128, seg_len <= 64): one
// workgroup per (batch, K/V head) walks all segments with (M, z) on chip.
bool fwd_short_supported(const Geometry& g);
hipError_t launch_fwd_short(const Geometry& g, const void* Q, const void* K, const void* V,
                            const float* beta, const float* M0, const float* z0, void* O,
                            float* M_S, float* z_S, float* lse, hipStream_t st);

// Fused short-segment backward (bf16, head_dim 64 or 128, seg_len <= 64,
// at most 16 query heads per K/V head).  dbeta_part: [B][Hq] scratch.  lse:
// the forward's row log-sum-exp [B][Hq][N], or NULL to form the softmax
// statistics again.  M_S_in, z_S_in: the forward's final state, or NULL to
// rebuild it from K, V, M0, z0.
bool bwd_short_supported(const Geometry& g);
hipError_t launch_bwd_short(const Geometry& g, const void* Q, const void* K, const void* V,
                            const float* beta, const float* M0, const float* z0, const void* dO,
                            const float* dM_S, const float* dz_S, void* dQ, void* dK, void* dV,
                            float* dbeta, float* dM0, float* dz0, float* dbeta_part, const float* lse,
                            hipStream_t st, const float* M_S_in = nullptr, const float* z_S_in = nullptr);

// Generic forward (fp32 vector arithmetic) over segments [s_begin, s_end),
// reading the per-segment snapshots written by launch_sweep.
// dst[i] = src ? src[i] : 0 for i < n.
hipError_t launch_state_copy(float* dst, const float* src, size_t n, hipStream_t st);

// Amem: when not NULL, the retrieved A_mem of every row ([B][Hq][nseg * L][D]
// fp32) is read from it instead of being formed from Msnap / zsnap.
hipError_t launch_fwd_generic(const Geometry& g, const void* Q, const void* K, const void* V,
                              const float* beta, const float* Msnap, const float* zsnap,
                              void* O, float* lse, int s_begin, int s_end, hipStream_t st,
                              const float* Amem = nullptr);

// Generic backward pieces, over segments [s_begin, s_end) (one chunk).
struct BwdChunkWs {
  float* lse;      // [B][Hq][C*L]
  float* Dd;       // [B][Hq][C*L]   rowsum(dA_dot * A_dot)
  float* dden;     // [B][Hq][C*L]
  float* dnum;     // [B][Hq][C*L][D]
  float* dbeta_part;  // [B][Hq][C][row blocks]
  float* dMsnap;   // [B*Hkv][C][D][D]   gradient w.r.t. M_s
  float* dzsnap;   // [B*Hkv][C][D]
};

int bwd_q_row_blocks(const Geometry& g);

// bf16 head_dim 64 / 128: the query- and key-side backward run on the matrix
// cores (bwd_long.hip), with the same workspace as the generic kernels.
bool bwd_long_mfma_supported(const Geometry& g);
int bwd_q_mfma_row_blocks(const Geometry& g);
// MhiT / MloT: the segments' M_{s-1} transposed, as bf16 and its bf16 rounding
// remainder ([B*Hkv][nseg][D][D], from launch_sweep_mfma).
hipError_t launch_bwd_q_mfma(const Geometry& g, const void* Q, const void* K, const void* V,
                             const float* beta, const void* MhiT, const void* MloT, const float* zsnap,
                             const void* dO, void* dQ, const BwdChunkWs& w, const float* lse_in, int s_begin,
                             int s_end, hipStream_t st);
// R, r: scratch [B*Hkv][nseg][D][D] and [B*Hkv][nseg][D] for the segments'
// retrieval terms; writes w.dMsnap / w.dzsnap and dM_out / dz_out as launch_rscan.
hipError_t launch_rscan_mfma(const Geometry& g, const void* Q, const BwdChunkWs& w, float* R, float* r,
                             const float* dM_in, const float* dz_in, float* dM_out, float* dz_out,
                             int s_begin, int s_end, hipStream_t st);
hipError_t launch_bwd_kv_mfma(const Geometry& g, const void* Q, const void* K, const void* V,
                              const float* beta, const void* dO, const BwdChunkWs& w, void* dK, void* dV,
                              int s_begin, int s_end, hipStream_t st);

// lse_in: the forward's row log-sum-exp [B][Hq][N] (the probabilities are
// then formed from it directly), or NULL to form it again.
hipError_t launch_bwd_q(const Geometry& g, const void* Q, const void* K, const void* V,
                        const float* beta, const float* Msnap, const float* zsnap,
                        const void* dO, void* dQ, const BwdChunkWs& w, const float* lse_in,
                        int s_begin, int s_end, hipStream_t st);

hipError_t launch_rscan(const Geometry& g, const void* Q, const BwdChunkWs& w,
                        const float* dM_in, const float* dz_in, float* dM_out, float* dz_out,
                        int s_begin, int s_end, hipStream_t st);

hipError_t launch_bwd_kv(const Geometry& g, const void* Q, const void* K, const void* V,
                         const float* beta, const void* dO, const BwdChunkWs& w,
                         void* dK, void* dV, int s_begin, int s_end, hipStream_t st);

// dbeta_acc[h] (=, or += unless first) sum of the chunk's partials; when last,
// dbeta[h] = g(1-g) * dbeta_acc[h].
hipError_t launch_dbeta_reduce(const Geometry& g, const float* beta, const BwdChunkWs& w,
                               float* dbeta_acc, float* dbeta, int nseg, bool first, bool last,
                               hipStream_t st);

// Streaming decode: Tn new rows at positions pos.. of the current segment;
// appends them to the caches Kc/Vc ([B*Hkv][L][D]) and writes O ([B][Hq][Tn][D]).
// `part` holds decode_partial_bytes(g, Tn) bytes for the key-split partials.
constexpr int kDecodeMaxSplits = 16;
size_t decode_partial_bytes(const Geometry& g, int Tn);
hipError_t launch_decode(const Geometry& g, int Tn, int pos, const void* Q, const void* K, const void* V,
                         const float* beta, void* Kc, void* Vc, const float* M, const float* z, void* O,
                         float* part, hipStream_t st);

}  // namespace infini
