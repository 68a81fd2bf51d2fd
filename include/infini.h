/*
 * libinfini — Infini-attention segment kernel for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes; no C++ or framework types.
 *
 * What is computed (per batch b, query head h, K/V head k = h / (Hq/Hkv)):
 * the sequence is cut into fixed-length segments of seg_len tokens (page
 * "Hugging Face Infini-Attention 재현 분석", section "Infini-Attention
 * 메커니즘", step Segmentation).  For segment s, with rows r:
 *
 *   A_dot = softmax(mask(Q_r K_r^T / sqrt(d))) V_r     causal, inside the segment
 *                                                       (same section, Local Attention)
 *   A_mem = sigma(Q_r) M_{s-1} / (sigma(Q_r) z_{s-1} + INFINI_MEM_EPS)
 *           sigma(x) = ELU(x) + 1 = x + 1 (x > 0), exp(x) (x <= 0)
 *                                                       (Memory Retrieval)
 *   O_r   = g_h A_mem + (1 - g_h) A_dot,  g_h = sigmoid(beta_h)   (Integration)
 *   M_s   = M_{s-1} + sigma(K_r)^T V_r,   z_s = z_{s-1} + sum_rows sigma(K_r)
 *                                                       (Memory Update)
 *
 * and only (M, z) is carried to the next segment (State Transfer).  When
 * seq_len is not a multiple of seg_len the last segment is shorter
 * (seq_len - (S-1) seg_len tokens, S = ceil(seq_len / seg_len)) and is
 * processed like the others; the pages fix the segment length but not what
 * happens to a remainder, so this is the reading taken.  The
 * normalised linear-attention form of A_mem follows the page
 * "[정보] KV선형 덧셈연산 인피니 어텐션에 대한 정보" (summary of "Leave No
 * Context Behind"), which calls the memory path long-term linear attention
 * that reuses the standard attention's query, key and value states.
 *
 * Layouts (all row-major, contiguous, device memory):
 *   Q, O, dQ, dO : [batch][q_heads][seq_len][head_dim]     dtype of the problem
 *   K, V, dK, dV : [batch][kv_heads][seq_len][head_dim]    dtype of the problem
 *   beta, dbeta  : [q_heads]                                float32
 *   M*, dM*      : [batch][kv_heads][D'][head_dim]          float32, M[a][c] = key-feature a, value c
 *   z*, dz*      : [batch][kv_heads][D']                    float32
 *                  (D' = head_dim for the default feature map; see
 *                  infini_feature_map_t)
 *   lse          : [batch][q_heads][seq_len]                float32, natural-log
 *                  log-sum-exp of each row's scaled local scores
 *
 * Alignment: every tensor pointer except beta, dbeta and lse, and every
 * workspace, must be 16-byte aligned (the kernels move 16-byte vectors);
 * a misaligned one is refused with INFINI_ERR_UNSUPPORTED.
 *
 * Ownership: the caller allocates and frees every buffer (inputs, outputs,
 * workspace).  The library never allocates, frees or synchronises; calls are
 * asynchronous on `stream` (a hipStream_t, NULL = the default stream).  The
 * only global state is the static per-device scratch of
 * infini_decode_noalloc (below); every other entry point keeps none, so
 * concurrent calls on different streams with disjoint buffers are safe;
 * calls sharing a workspace (or that scratch) must be ordered by the caller.
 *
 * Errors: arguments are validated on the host before anything is launched;
 * on a validation error nothing is written.  INFINI_ERR_HIP reports a failed
 * launch; launches of the same call issued before it may have run, so the
 * outputs are then unspecified.
 */
#ifndef INFINI_H
#define INFINI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Added to sigma(Q) z in the retrieval denominator.  With an empty memory
 * (M0 = z0 = 0) it makes A_mem exactly 0 in the first segment instead of 0/0. */
#define INFINI_MEM_EPS 1e-6f

#define INFINI_VERSION 2

typedef enum {
  INFINI_OK = 0,
  INFINI_ERR_NULL = 1,        /* a required pointer is NULL                                   */
  INFINI_ERR_SHAPE = 2,       /* a negative batch or seq_len, another dim <= 0, or
                                 q_heads % kv_heads != 0                                       */
  INFINI_ERR_UNSUPPORTED = 3, /* head_dim not 32, 64 or 128, unknown dtype or feature map, a
                                 feature map the entry point does not support, or a tensor
                                 pointer (any but beta, dbeta, lse) not 16-byte aligned        */
  INFINI_ERR_ALIAS = 4,       /* an output buffer overlaps an input or another output          */
  INFINI_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the size query returns          */
  INFINI_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed                      */
  INFINI_ERR_SCRATCH = 7      /* infini_decode_noalloc: the problem needs more scratch than
                                 INFINI_NOALLOC_SCRATCH_BYTES                                  */
} infini_status_t;

typedef enum { INFINI_FP32 = 0, INFINI_BF16 = 1 } infini_dtype_t;

/* Feature map of the memory path.
 *   INFINI_FEATURE_ELU1     sigma(x) = ELU(x) + 1 elementwise; M is
 *                           [head_dim][head_dim], z has head_dim entries.
 *   INFINI_FEATURE_TAYLOR2  the second-order Taylor map of the page "Based"
 *                           (cartesia.ai), section "고정 크기 순환 상태를 사용하는
 *                           방법도 중요합니다": phi(x) = [1, x_1..x_d,
 *                           x_a x_b / sqrt(2) for a, b = 1..d, a major], so that
 *                           phi(q) . phi(k) = 1 + q.k + (q.k)^2 / 2, applied to
 *                           Q and K as given.  D' = 1 + d + d^2 features: M is
 *                           [D'][head_dim], z has D' entries, row f of M holding
 *                           feature f.  Supported by infini_attn_fwd and
 *                           infini_attn_fwd_varlen, every dtype and head_dim;
 *                           every other entry point returns
 *                           INFINI_ERR_UNSUPPORTED for it.  bf16 with head_dim
 *                           64 or 128 and seq_len <= 16 D' runs on the matrix
 *                           cores without forming any per-segment state: the
 *                           retrieval for a query of segment s is the
 *                           attention over the keys before the segment with
 *                           weights 1 + q.k + (q.k)^2 / 2, plus phi(q) M0 and
 *                           phi(q) z0 for a starting state, which equals
 *                           phi(q) M_{s-1} / (phi(q) z_{s-1} + eps); other
 *                           calls take fp32 vector kernels over the D'-row
 *                           states. */
typedef enum { INFINI_FEATURE_ELU1 = 0, INFINI_FEATURE_TAYLOR2 = 1 } infini_feature_map_t;

/* One call's problem.  The carried state is always float32.
 *
 * Empty problems: batch = 0 or seq_len = 0 is valid for every entry point
 * except infini_decode.  Nothing is computed: a forward hands the state through
 * (M_S = M0, z_S = z0, zeros when they are NULL; infini_fwd_stream leaves M and
 * z as they are), a backward writes dbeta = 0 and dM0 = dM_S, dz0 = dz_S
 * (zeros when NULL).  Pointers to tensors of no elements may be NULL, and a
 * workspace of 0 bytes may be NULL. */
typedef struct {
  int32_t batch;
  int32_t q_heads;
  int32_t kv_heads;   /* q_heads % kv_heads == 0; query head h reads K/V head h / (q_heads/kv_heads) */
  int32_t seq_len;    /* tokens in this call; the last segment may be shorter than seg_len         */
  int32_t head_dim;   /* 32, 64 or 128; keys, queries and values share it                            */
  int32_t seg_len;    /* tokens per segment                                                          */
  int32_t dtype;      /* infini_dtype_t of Q, K, V, O, dO, dQ, dK, dV                                */
  int32_t feature_map; /* infini_feature_map_t of the memory path (0 = ELU + 1)                      */
} infini_problem_t;

/* Workspace bytes for infini_attn_fwd.  Bounded by a constant times
 * batch*kv_heads*head_dim^2 that does not grow with seq_len (segments are
 * processed in chunks of at most a fixed number).  Returns 0 for an invalid
 * problem. */
size_t infini_fwd_workspace_bytes(const infini_problem_t* p);

/* Workspace bytes for infini_attn_bwd (does not grow with seq_len either;
 * on the fused short-segment path only batch * q_heads floats). */
size_t infini_bwd_workspace_bytes(const infini_problem_t* p);

/* Bytes of what the forward saves for the backward: its optional lse output,
 * batch * q_heads * seq_len floats (the natural-log log-sum-exp of every
 * row's scaled causal scores inside its segment).  Nothing else needs to be
 * kept: the backward recomputes the attention probabilities from Q, K and
 * this row statistic, and the state from K, V, M0 and z0.  0 for an invalid
 * problem. */
size_t infini_fwd_saved_bytes(const infini_problem_t* p);

/* Forward.
 *   Q, K, V   inputs (layouts above)
 *   beta      [q_heads] gate parameters
 *   M0, z0    carried state from an earlier call, or both NULL for an empty
 *             memory.  Precondition: either both zero/NULL or produced by an
 *             earlier call (or a consistent sum sigma(K)^T V, sum sigma(K));
 *             z0 = 0 with M0 != 0 gives unspecified results.
 *   O         [batch][q_heads][seq_len][head_dim] output
 *   M_S, z_S  state after the last segment (must not alias M0 / z0: chained
 *             calls ping-pong between two state buffers)
 *   lse       optional [batch][q_heads][seq_len] float32 output (the saved
 *             buffer, infini_fwd_saved_bytes(p) bytes), for the backward;
 *             NULL to skip
 *   ws        device workspace of at least infini_fwd_workspace_bytes(p); on
 *             the fused short-segment path (infini_fwd_path(p) returns
 *             "mfma_bf16_short"), and on the matrix-core Taylor path
 *             ("mfma_bf16_taylor2") when M0 is NULL, the call uses none and
 *             ws may be NULL with ws_bytes 0 (the size query still returns
 *             what the other paths need for the same problem); with M0 the
 *             matrix-core Taylor path uses batch * q_heads * seq_len *
 *             (head_dim + 1) floats of it
 */
infini_status_t infini_attn_fwd(const infini_problem_t* p,
                                const void* Q, const void* K, const void* V,
                                const float* beta, const float* M0, const float* z0,
                                void* O, float* M_S, float* z_S, float* lse,
                                void* ws, size_t ws_bytes, void* stream);

/* Backward: the exact gradient of infini_attn_fwd for
 *   loss = <dO, O> + <dM_S, M_S> + <dz_S, z_S>.
 *   Q, K, V, beta, M0, z0   the forward's inputs (M0, z0 both NULL = empty memory)
 *   lse        the forward's lse output for the same inputs, or NULL.  When
 *              given, the attention probabilities are formed from it directly
 *              (exp(score - lse): no running row maximum, no row sum); when
 *              NULL those statistics are formed again.  Either way the
 *              gradients agree within rounding; an lse that does not belong
 *              to these inputs gives unspecified gradients (no fault).
 *   dO         upstream gradient of O (dtype of the problem)
 *   dM_S, dz_S upstream gradients of the final state, or NULL for zero
 *   dQ, dK, dV gradients (dtype of the problem), overwritten
 *   dbeta      [q_heads] float32, overwritten
 *   dM0, dz0   gradients of the state passed in, or NULL to skip; chaining
 *              them as dM_S, dz_S of the previous call backpropagates through
 *              a sequence of calls
 *   ws         device workspace of at least infini_bwd_workspace_bytes(p)
 */
infini_status_t infini_attn_bwd(const infini_problem_t* p,
                                const void* Q, const void* K, const void* V,
                                const float* beta, const float* M0, const float* z0,
                                const float* lse, const void* dO,
                                const float* dM_S, const float* dz_S,
                                void* dQ, void* dK, void* dV, float* dbeta,
                                float* dM0, float* dz0,
                                void* ws, size_t ws_bytes, void* stream);

/* Backward with the state the forward returned.  Arguments as for
 * infini_attn_bwd_varlen (seq_lens NULL = every sequence has seq_len tokens),
 * plus
 *   M_S, z_S   the forward's M_S, z_S for the same inputs (read only; both
 *              non-NULL, or both NULL for exactly infini_attn_bwd_varlen).
 * The backward walks the segments from last to first and needs the state
 * after the last one: given here, it is not rebuilt from K, V, M0, z0 (one
 * pass over K and V less on the fused short-segment path; a copy instead of a
 * memory sweep on the chunked paths).  The gradients equal those of
 * infini_attn_bwd within rounding when M_S, z_S are the forward's outputs
 * (on the fused short-segment path they are the same state bit for bit); a
 * state that does not belong to these inputs gives unspecified gradients (no
 * fault).  This is the other half of the saved-state contract: a training
 * step keeps lse (infini_fwd_saved_bytes) and the final state it returns
 * anyway. */
infini_status_t infini_attn_bwd_saved(const infini_problem_t* p, const int32_t* seq_lens,
                                      const void* Q, const void* K, const void* V,
                                      const float* beta, const float* M0, const float* z0,
                                      const float* M_S, const float* z_S,
                                      const float* lse, const void* dO,
                                      const float* dM_S, const float* dz_S,
                                      void* dQ, void* dK, void* dV, float* dbeta,
                                      float* dM0, float* dz0,
                                      void* ws, size_t ws_bytes, void* stream);

/* Variable-length batches: the forward and backward above for a batch whose
 * sequences have different lengths (page "Hugging Face Infini-Attention 재현
 * 분석", section "Infini-Attention 메커니즘", step Segmentation, applied to
 * each sequence on its own).
 *   seq_lens  device int32 [batch]: sequence b holds seq_lens[b] tokens in
 *             rows 0 .. seq_lens[b]-1 of its seq_len-row slot (p->seq_len is
 *             the capacity, the longest sequence); 4-byte aligned.  Values
 *             are read on the device, so they cannot be checked before the
 *             launch: each is clamped to [0, p->seq_len].  NULL = every
 *             sequence has p->seq_len tokens (then identical to the calls
 *             above).
 * Each sequence is cut into its own segments, the last possibly shorter, and
 * processed exactly as if it were alone: its state M_S[b], z_S[b] is the one
 * after its own last segment (M0[b], z0[b] for an empty sequence), and dbeta
 * sums over the sequences.  Rows past a sequence's end are never read, and
 * are written as zeros in O, lse, dQ, dK and dV.  Workspace sizes are those of
 * the same problem without seq_lens; every other argument, layout and error
 * is as for infini_attn_fwd / infini_attn_bwd. */
infini_status_t infini_attn_fwd_varlen(const infini_problem_t* p, const int32_t* seq_lens,
                                       const void* Q, const void* K, const void* V,
                                       const float* beta, const float* M0, const float* z0,
                                       void* O, float* M_S, float* z_S, float* lse,
                                       void* ws, size_t ws_bytes, void* stream);
infini_status_t infini_attn_bwd_varlen(const infini_problem_t* p, const int32_t* seq_lens,
                                       const void* Q, const void* K, const void* V,
                                       const float* beta, const float* M0, const float* z0,
                                       const float* lse, const void* dO,
                                       const float* dM_S, const float* dz_S,
                                       void* dQ, void* dK, void* dV, float* dbeta,
                                       float* dM0, float* dz0,
                                       void* ws, size_t ws_bytes, void* stream);

/* Segments whose per-segment state a workspace holds at once.  Longer calls
 * are processed in chunks of this many segments. */
#define INFINI_CHUNK_SEGMENTS 16

/* The forward in its two phases, for callers that schedule them separately
 * (for example to overlap the memory phase of one layer with the attention
 * phase of another, or to time each phase).  Only for calls with at most
 * INFINI_CHUNK_SEGMENTS segments (ceil(seq_len / seg_len)); longer calls return
 * INFINI_ERR_SHAPE and must use infini_attn_fwd.
 *
 * infini_fwd_memory runs the memory path alone (same page and section,
 * steps Memory Update and State Transfer): it writes M_S, z_S and leaves in
 * `ws` the state each segment retrieves from.  infini_fwd_attend then runs
 * local attention, retrieval and the gate for every segment, reading that
 * state from `ws`; between the two calls the caller must not touch `ws`.
 * Running both with the same arguments as infini_attn_fwd gives bit-identical
 * results.  Argument meanings, layouts and errors are those of
 * infini_attn_fwd. */
infini_status_t infini_fwd_memory(const infini_problem_t* p, const void* K, const void* V,
                                  const float* M0, const float* z0, float* M_S, float* z_S,
                                  void* ws, size_t ws_bytes, void* stream);
infini_status_t infini_fwd_attend(const infini_problem_t* p, const void* Q, const void* K,
                                  const void* V, const float* beta, void* O, float* lse,
                                  const void* ws, size_t ws_bytes, void* stream);

/* Streaming forward: n_launches consecutive calls of shape *p (each at most
 * INFINI_CHUNK_SEGMENTS segments; a call whose seq_len is not a multiple of
 * seg_len ends in a shorter segment, as in infini_attn_fwd), the state carried from
 * one call to the next (page "Hugging Face Infini-Attention 재현 분석",
 * section "Infini-Attention 메커니즘", step State Transfer), issued so that
 * they overlap.  The calls go in groups of `group`: the memory phases
 * (infini_fwd_memory) run in order on mem_stream, and once a group's memory
 * phases are done its attention phases (infini_fwd_attend) run on
 * att_streams[k % n_pipe] for group k.  Where the problem takes the
 * matrix-core path a group's memory phases are one run over the group's
 * segments and its attention phases one launch (then group * segments per
 * call may not exceed INFINI_CHUNK_SEGMENTS).  Outputs and final
 * state are bit-identical to n_launches chained infini_attn_fwd calls.
 *   Q, K, V, O   host arrays of n_launches device pointers; call i uses Q[i],
 *                K[i], V[i] and writes O[i], with the layouts of infini_attn_fwd
 *   beta         [q_heads] float32
 *   M, z         [batch][kv_heads][head_dim][head_dim] and [batch][kv_heads]
 *                [head_dim] float32: the state before call 0 on entry, updated
 *                in place by the memory phases on mem_stream
 *   ws           infini_fwd_stream_workspace_bytes(p, n_pipe, group) bytes
 *                (ws_bytes: its size)
 *   n_pipe       groups in flight (>= 1); group: calls per group, 1 to
 *                INFINI_STREAM_MAX_GROUP
 *   mem_stream   stream of the memory phases; att_streams: n_pipe streams for
 *                the attention phases; events: 2 * n_pipe events of the
 *                caller's (timing may be disabled), used to order the phases
 * Inputs must be ready on every stream passed; the call returns once all work
 * is issued, and the caller orders later work after mem_stream and all
 * att_streams.  The schedule cannot be recorded into a HIP graph: if
 * mem_stream or an attention stream is being captured the call returns
 * INFINI_ERR_UNSUPPORTED and issues nothing (chained infini_attn_fwd calls
 * on one stream can be captured).  Errors are those of infini_attn_fwd, plus INFINI_ERR_SHAPE
 * for n_launches < 1, n_pipe < 1, group outside [1, INFINI_STREAM_MAX_GROUP],
 * more than INFINI_CHUNK_SEGMENTS segments per call, or (matrix-core path)
 * per group; arguments are all
 * checked before anything is issued.  One library call per batch of calls,
 * and two events per group rather than per call, keep the host's issue cost
 * per call low. */
#define INFINI_STREAM_MAX_GROUP 8
/* Workspace bytes for infini_fwd_stream; 0 for an invalid problem or
 * arguments. */
size_t infini_fwd_stream_workspace_bytes(const infini_problem_t* p, int n_pipe, int group);
infini_status_t infini_fwd_stream(const infini_problem_t* p, int n_launches, const void* const* Q,
                                  const void* const* K, const void* const* V, const float* beta,
                                  float* M, float* z, void* const* O, void* ws, size_t ws_bytes,
                                  int n_pipe, int group, void* mem_stream, void* const* att_streams,
                                  void* const* events);

/* Streaming decode: a few new tokens of the segment that is being filled.
 *
 * The same computation as infini_attn_fwd, evaluated for the tokens a
 * generation loop produces one (or a few) at a time (page "Hugging Face
 * Infini-Attention 재현 분석", section "Infini-Attention 메커니즘": Local
 * Attention, Memory Retrieval, Integration, and Memory Update once the
 * segment is complete).  Feeding a sequence through infini_decode in pieces
 * gives the outputs and the state of one infini_attn_fwd call over it.
 *
 *   p->seq_len   T, the new tokens of this call (>= 1)
 *   p->seg_len   L; other fields as for infini_attn_fwd
 *   pos          tokens of the current segment already in the caches,
 *                0 <= pos and pos + T <= L
 *   Q            [B][Hq][T][d] new query rows
 *   K, V         [B][Hkv][T][d] new key and value rows
 *   Kcache, Vcache  [B][Hkv][L][d], caller-owned, in/out: rows [0, pos) hold
 *                the segment's earlier tokens; this call writes rows
 *                [pos, pos + T).  Rows past pos + T are not read.
 *   M, z         state before the current segment ([B][Hkv][d][d],
 *                [B][Hkv][d] fp32; both NULL = empty memory)
 *   O            [B][Hq][T][d] output rows (row t is token pos + t)
 *   M_next, z_next  written only when pos + T == L (the call completes the
 *                segment): the state after it, M + sigma(Kcache)^T Vcache
 *                and z + sum_rows sigma(Kcache); may be NULL otherwise
 *   ws, ws_bytes    infini_decode_workspace_bytes(p) bytes of scratch, on
 *                every call (key-split partials of the rows, and the memory
 *                update when the call completes the segment); it depends on
 *                T and the shape, not on pos
 *
 * Errors: INFINI_ERR_SHAPE for T < 1, batch < 1, pos < 0 or pos + T > L (and
 * the shape checks of infini_attn_fwd); INFINI_ERR_NULL for a missing pointer, a half-given
 * state, or a missing M_next/z_next on the completing call;
 * INFINI_ERR_WORKSPACE; INFINI_ERR_ALIAS when O, the caches, M_next, z_next
 * or ws overlap an input or each other.  Calls are asynchronous on stream. */
size_t infini_decode_workspace_bytes(const infini_problem_t* p);
infini_status_t infini_decode(const infini_problem_t* p, int32_t pos, const void* Q, const void* K,
                              const void* V, const float* beta, void* Kcache, void* Vcache,
                              const float* M, const float* z, void* O, float* M_next, float* z_next,
                              void* ws, size_t ws_bytes, void* stream);

/* Allocation-free streaming decode, for callers that cannot allocate device
 * memory: code recorded under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.  Arguments, results and errors are those
 * of infini_decode, without the workspace: the scratch comes from a static
 * per-device array of INFINI_NOALLOC_SCRATCH_BYTES that the library holds
 * for the life of the process (set up, without allocating, on the first call
 * made with each device current; stream must belong to the current device).
 * A problem whose infini_decode_workspace_bytes exceeds that size returns
 * INFINI_ERR_SCRATCH before anything is issued.  Every call on a device
 * shares that device's array, and no value in it survives from one call to
 * the next that a later call reads; calls on one device whose executions
 * overlap (different streams, not ordered by the caller) race on it and
 * give unspecified results.  The call itself allocates and frees nothing. */
#define INFINI_NOALLOC_SCRATCH_BYTES (32u << 20)
infini_status_t infini_decode_noalloc(const infini_problem_t* p, int32_t pos, const void* Q, const void* K,
                                      const void* V, const float* beta, void* Kcache, void* Vcache,
                                      const float* M, const float* z, void* O, float* M_next, float* z_next,
                                      void* stream);

/* Name of the kernel family infini_attn_fwd runs for this problem
 * ("generic_fp32": fp32 vector-ALU path; "mfma_bf16": bf16 matrix-core
 * path, memory phase then attention phase; "mfma_bf16_short": bf16
 * matrix-core path for seg_len <= 64 that keeps the memory on chip in one
 * fused kernel; with the Taylor feature map "mfma_bf16_taylor2", the
 * matrix-core Taylor path, or "generic_fp32_taylor2", the fp32 vector
 * kernels).  NULL for an invalid problem.  Static storage. */
const char* infini_fwd_path(const infini_problem_t* p);

/* Static description of a status code. */
const char* infini_status_string(infini_status_t s);

/* INFINI_VERSION of the loaded library. */
int infini_version(void);

#ifdef __cplusplus
}
#endif

#endif /* INFINI_H */
