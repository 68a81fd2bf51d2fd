// Memory path with the second-order Taylor feature map (fp32 vector ALU).
//
// Page "Based" (cartesia.ai), section "고정 크기 순환 상태를 사용하는 방법도
// 중요합니다": the feature map phi is chosen so that phi(q) . phi(k) is the
// second-order Taylor series of exp(q . k), 1 + q.k + (q.k)^2 / 2, and the
// key dimension grows from d to about d^2.  Here
//   phi(x) = [1, x_1 .. x_d, x_a x_b / sqrt 2 (a major)],  D' = 1 + d + d^2,
// applied to Q and K as they arrive.  It replaces sigma = ELU + 1 in the
// memory path of page "Hugging Face Infini-Attention 재현 분석", section
// "Infini-Attention 메커니즘" (Memory Retrieval, Memory Update, State
// Transfer); local attention and the gate are unchanged:
//   M_s = M_{s-1} + phi(K_s)^T V_s   (D' x d),   z_s = z_{s-1} + sum_rows phi(K_s)
//   A_mem = phi(Q) M_{s-1} / (phi(Q) z_{s-1} + eps)
//
//   taylor_sweep_kernel     one workgroup per 32x32 tile of M (features x
//                           values) per (batch, K/V head): walks the segments
//                           in order, writes each M_{s-1}, z_{s-1} and
//                           accumulates phi(K)^T V; the features of a staged
//                           key chunk are formed in LDS from whole key rows.
//   taylor_retrieve_kernel  one workgroup per 32 query rows of a (batch,
//                           query head, segment): M_{s-1} streamed through
//                           LDS d feature rows at a time (the constant and
//                           linear rows, then quadratic row a, whose features
//                           are q_a q_b / sqrt 2), A_mem written in fp32 for
//                           the attention kernel's gate.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace infini {

constexpr float kRsqrt2 = 0.70710678118654752f;
constexpr int TS_TILE = 32;      // sweep tile edge (features and value columns)
constexpr int TS_KEYS = 32;      // keys staged per step
constexpr int TR_ROWS = 32;      // query rows per retrieval workgroup

size_t taylor_dim(int D) { return 1 + (size_t)D + (size_t)D * D; }

// Feature f (< 1 + D + D^2) of the row x (D floats).
template <int D>
__device__ __forceinline__ float taylor_feature(const float* x, int f) {
  if (f == 0) return 1.f;
  if (f <= D) return x[f - 1];
  const int r = f - 1 - D;
  return x[r / D] * x[r % D] * kRsqrt2;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void taylor_sweep_kernel(
    const T* __restrict__ K, const T* __restrict__ V, const float* M_in, const float* z_in, float* M_out,
    float* z_out, float* __restrict__ Msnap, float* __restrict__ zsnap, int N, int L, int s_begin, int s_end,
    const int* __restrict__ lens, int Hkv) {
  constexpr int DF = 1 + D + D * D;
  constexpr int CT = D / TS_TILE;                  // value-column tiles
  const int f0 = (blockIdx.x / CT) * TS_TILE;
  const int c0 = (blockIdx.x % CT) * TS_TILE;
  const bool do_z = (blockIdx.x % CT) == 0;
  const size_t bh = blockIdx.y;
  const int t = threadIdx.x;
  const int ta = t >> 3;                           // feature row in the tile, 0..31
  const int tc = (t & 7) * 4;                      // 4 value columns
  const bool frow = f0 + ta < DF;
  const bool z_lane = do_z && t < TS_TILE && f0 + t < DF;

  __shared__ float sKr[TS_KEYS][D + 1];            // whole key rows of the chunk
  __shared__ float sPhi[TS_KEYS][TS_TILE + 1];     // the tile's features of each key
  __shared__ float sV[TS_KEYS][TS_TILE + 4];

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float zacc = 0.f;
  const size_t mrow = bh * DF * D + (size_t)(f0 + ta) * D + c0 + tc;
  if (frow)
    for (int c = 0; c < 4; ++c) acc[c] = M_in ? M_in[mrow + c] : 0.f;
  if (z_lane) zacc = z_in ? z_in[bh * DF + f0 + t] : 0.f;

  const int nseg = s_end - s_begin;
  const int Nb = seq_len_of(lens, (int)(bh / Hkv), N);
  for (int s = s_begin; s < s_end; ++s) {
    const size_t snap = bh * nseg + (s - s_begin);
    if (frow)
      for (int c = 0; c < 4; ++c) Msnap[(snap * DF + f0 + ta) * D + c0 + tc + c] = acc[c];
    if (z_lane) zsnap[snap * DF + f0 + t] = zacc;
    const size_t rowbase = (bh * N + (size_t)s * L) * D;
    const int Ls = min(L, Nb - s * L);             // keys of this segment (none past the sequence's end)
    for (int j0 = 0; j0 < Ls; j0 += TS_KEYS) {
      const int jn = min(TS_KEYS, Ls - j0);
      for (int e = t; e < TS_KEYS * D; e += 256) {
        const int j = e / D, a = e % D;
        sKr[j][a] = j < jn ? io<T>::load(K, rowbase + (size_t)(j0 + j) * D + a) : 0.f;
      }
      for (int e = t; e < TS_KEYS * TS_TILE; e += 256) {
        const int j = e / TS_TILE, x = e % TS_TILE;
        sV[j][x] = j < jn ? io<T>::load(V, rowbase + (size_t)(j0 + j) * D + c0 + x) : 0.f;
      }
      __syncthreads();
      for (int e = t; e < TS_KEYS * TS_TILE; e += 256) {
        const int j = e / TS_TILE, x = e % TS_TILE;
        sPhi[j][x] = (j < jn && f0 + x < DF) ? taylor_feature<D>(sKr[j], f0 + x) : 0.f;
      }
      __syncthreads();
      for (int j = 0; j < jn; ++j) {
        const float p = sPhi[j][ta];
        for (int c = 0; c < 4; ++c) acc[c] += p * sV[j][tc + c];
        if (z_lane) zacc += sPhi[j][t];
      }
      __syncthreads();
    }
  }
  if (M_out) {
    if (frow)
      for (int c = 0; c < 4; ++c) M_out[mrow + c] = acc[c];
    if (z_lane) z_out[bh * DF + f0 + t] = zacc;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void taylor_retrieve_kernel(
    const T* __restrict__ Q, const float* __restrict__ Msnap, const float* __restrict__ zsnap,
    float* __restrict__ Amem, int Hq, int Hkv, int N, int L, int s_begin, int nseg,
    const int* __restrict__ lens) {
  constexpr int DF = 1 + D + D * D;
  constexpr int CPT = D / 8;                       // value columns per thread
  __shared__ float sQ[TR_ROWS][D + 1];
  __shared__ float sM[D][D];                       // d feature rows of M_{s-1}
  __shared__ float sz[D];
  __shared__ float sM0[D];                         // the constant feature's row
  __shared__ float sz0;

  const int t = threadIdx.x;
  const int r = t >> 3;                            // query row of the block
  const int cg = t & 7;                            // column group
  const int h = blockIdx.y;
  const int sl = blockIdx.z % nseg;
  const int b = blockIdx.z / nseg;
  const int s = s_begin + sl;
  const int kvh = h / (Hq / Hkv);
  const int Ls = min(L, seq_len_of(lens, b, N) - s * L);
  const int i0 = blockIdx.x * TR_ROWS;
  if (i0 >= Ls) return;                            // rows past the segment (or the sequence)
  const size_t qbase = (((size_t)b * Hq + h) * N + (size_t)s * L) * D;
  for (int e = t; e < TR_ROWS * D; e += 256) {
    const int rr = e / D, a = e % D;
    sQ[rr][a] = i0 + rr < Ls ? io<T>::load(Q, qbase + (size_t)(i0 + rr) * D + a) : 0.f;
  }
  const size_t snap = (size_t)(b * Hkv + kvh) * nseg + sl;
  const float* Ms = Msnap + snap * DF * D;
  const float* zz = zsnap + snap * DF;
  float num[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) num[c] = 0.f;
  float den = 0.f;
  // chunk -1: the constant row 0 and the linear rows 1..D (features 1, q_b);
  // chunk a: quadratic rows 1 + D + a D + b (features q_a q_b / sqrt 2)
  for (int ch = -1; ch < D; ++ch) {
    const size_t first = ch < 0 ? 1 : 1 + D + (size_t)ch * D;
    for (int e = t; e < D * D; e += 256) sM[e / D][e % D] = Ms[(first + e / D) * D + e % D];
    for (int e = t; e < D; e += 256) sz[e] = zz[first + e];
    if (ch < 0) {
      for (int e = t; e < D; e += 256) sM0[e] = Ms[e];
      if (t == 0) sz0 = zz[0];
    }
    __syncthreads();
    if (ch < 0) {
      den += sz0;
#pragma unroll
      for (int c = 0; c < CPT; ++c) num[c] += sM0[cg * CPT + c];
    }
    const float w = ch < 0 ? 1.f : sQ[r][ch] * kRsqrt2;
    for (int bb = 0; bb < D; ++bb) {
      const float phi = w * sQ[r][bb];
      den += phi * sz[bb];
#pragma unroll
      for (int c = 0; c < CPT; ++c) num[c] += phi * sM[bb][cg * CPT + c];
    }
    __syncthreads();
  }
  const int i = i0 + r;
  if (i < Ls) {
    const float inv = 1.f / (den + 1e-6f);
    float* out = Amem + (((size_t)b * Hq + h) * ((size_t)nseg * L) + (size_t)sl * L + i) * D + cg * CPT;
#pragma unroll
    for (int c = 0; c < CPT; ++c) out[c] = num[c] * inv;
  }
}

#define TAYLOR_DISPATCH(FN, ...)                                   \
  do {                                                              \
    if (g.dtype == 0) {                                             \
      if (g.D == 32) return FN<float, 32>(__VA_ARGS__);             \
      if (g.D == 64) return FN<float, 64>(__VA_ARGS__);             \
      if (g.D == 128) return FN<float, 128>(__VA_ARGS__);           \
    } else {                                                        \
      if (g.D == 32) return FN<bf16_t, 32>(__VA_ARGS__);            \
      if (g.D == 64) return FN<bf16_t, 64>(__VA_ARGS__);            \
      if (g.D == 128) return FN<bf16_t, 128>(__VA_ARGS__);          \
    }                                                               \
    return hipErrorInvalidValue;                                    \
  } while (0)

template <typename T, int D>
static hipError_t taylor_sweep_t(const Geometry& g, const void* K, const void* V, const float* M_in,
                                 const float* z_in, float* M_out, float* z_out, float* Msnap, float* zsnap,
                                 int s_begin, int s_end, hipStream_t st) {
  constexpr int DF = 1 + D + D * D;
  dim3 grid(((DF + TS_TILE - 1) / TS_TILE) * (D / TS_TILE), g.B * g.Hkv);
  hipLaunchKernelGGL((taylor_sweep_kernel<T, D>), grid, dim3(256), 0, st, static_cast<const T*>(K),
                     static_cast<const T*>(V), M_in, z_in, M_out, z_out, Msnap, zsnap, g.N, g.L, s_begin, s_end,
                     g.lens, g.Hkv);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t taylor_retrieve_t(const Geometry& g, const void* Q, const float* Msnap, const float* zsnap,
                                    float* Amem, int s_begin, int s_end, hipStream_t st) {
  const int nseg = s_end - s_begin;
  dim3 grid((g.L + TR_ROWS - 1) / TR_ROWS, g.Hq, g.B * nseg);
  hipLaunchKernelGGL((taylor_retrieve_kernel<T, D>), grid, dim3(256), 0, st, static_cast<const T*>(Q), Msnap,
                     zsnap, Amem, g.Hq, g.Hkv, g.N, g.L, s_begin, nseg, g.lens);
  return hipGetLastError();
}

hipError_t launch_taylor_sweep(const Geometry& g, const void* K, const void* V, const float* M_in,
                               const float* z_in, float* M_out, float* z_out, float* Msnap, float* zsnap,
                               int s_begin, int s_end, hipStream_t st) {
  TAYLOR_DISPATCH(taylor_sweep_t, g, K, V, M_in, z_in, M_out, z_out, Msnap, zsnap, s_begin, s_end, st);
}

hipError_t launch_taylor_retrieve(const Geometry& g, const void* Q, const float* Msnap, const float* zsnap,
                                  float* Amem, int s_begin, int s_end, hipStream_t st) {
  TAYLOR_DISPATCH(taylor_retrieve_t, g, Q, Msnap, zsnap, Amem, s_begin, s_end, st);
}

}  // namespace infini
