// Memory sweep and generic forward of the Infini-attention segment kernel.
//
// The memory path (page "Hugging Face Infini-Attention 재현 분석", section
// "Infini-Attention 메커니즘", steps Memory Update and State Transfer) is a
// prefix sum over segments of sigma(K_s)^T V_s and sum_rows sigma(K_s): it
// depends on K and V only.  `sweep_kernel` walks the segments in order with a
// tile of M resident in registers and publishes, for every segment, the state
// that segment retrieves from (M_{s-1}, z_{s-1}); the attention kernels then
// run all segments in parallel.
//
// `fwd_generic_kernel` is the plain fp32 vector-ALU forward used for fp32
// problems and as the always-available path: one query row per lane (two
// lanes per row at head_dim 128), K/V tiles staged in LDS, the online-softmax
// merge of per-tile row maxima and sums (page "Context Memorization for
// Efficient Long Context Generation", section "방법론": attention states over
// key sub-blocks merge exactly), then retrieval and the gate fused in the
// epilogue.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace infini {

// ---------------------------------------------------------------- sweep

constexpr int SW_TILE = 32;      // 32 x 32 tile of M per workgroup
constexpr int SW_KEYS = 64;      // keys staged per step

template <typename T, int D>
__global__ __launch_bounds__(256) void sweep_kernel(
    const T* __restrict__ K, const T* __restrict__ V,
    const float* M_in, const float* z_in, float* M_out, float* z_out,
    float* __restrict__ Msnap, float* __restrict__ zsnap, bf16_t* __restrict__ MsnapT,
    int N, int L, int s_begin, int s_end, const int* __restrict__ lens, int Hkv, float sign) {
  constexpr int TPR = D / SW_TILE;                 // tiles per row of M
  const int tile = blockIdx.x;
  const int a0 = (tile / TPR) * SW_TILE;
  const int c0 = (tile % TPR) * SW_TILE;
  const bool do_z = (tile % TPR) == 0;
  const size_t bh = blockIdx.y;
  const int t = threadIdx.x;
  const int ta = t >> 3;                           // row in tile, 0..31
  const int tc = (t & 7) * 4;                      // 4 columns

  __shared__ float sK[SW_KEYS][SW_TILE + 1];
  __shared__ float sV[SW_KEYS][SW_TILE + 4];

  float acc[4];
  float zacc = 0.f;
  const size_t mbase = bh * D * D + (size_t)(a0 + ta) * D + c0 + tc;
  for (int c = 0; c < 4; ++c) acc[c] = M_in ? M_in[mbase + c] : 0.f;
  const bool z_lane = do_z && t < SW_TILE;
  if (z_lane) zacc = z_in ? z_in[bh * D + a0 + t] : 0.f;

  const int nseg = s_end - s_begin;
  for (int s = s_begin; s < s_end; ++s) {
    if (Msnap) {
      const size_t sb = (bh * nseg + (s - s_begin)) * (size_t)D * D + (size_t)(a0 + ta) * D + c0 + tc;
      for (int c = 0; c < 4; ++c) Msnap[sb + c] = acc[c];
      if (z_lane) zsnap[(bh * nseg + (s - s_begin)) * D + a0 + t] = zacc;
    }
    if (MsnapT) {
      const size_t tb = (bh * nseg + (s - s_begin)) * (size_t)D * D;
      for (int c = 0; c < 4; ++c) MsnapT[tb + (size_t)(c0 + tc + c) * D + a0 + ta] = f32_to_bf16(acc[c]);
    }
    const size_t rowbase = (bh * N + (size_t)s * L) * D;
    // keys of this segment: the last may be short, and in a variable-length
    // batch the segment may lie past its sequence's end (no keys)
    const int Ls = min(L, seq_len_of(lens, (int)(bh / Hkv), N) - s * L);
    for (int j0 = 0; j0 < Ls; j0 += SW_KEYS) {
      for (int e = t; e < SW_KEYS * SW_TILE; e += 256) {
        const int j = e / SW_TILE, x = e % SW_TILE;
        float kv = 0.f, vv = 0.f;
        if (j0 + j < Ls) {
          const size_t gi = rowbase + (size_t)(j0 + j) * D;
          kv = elu1(io<T>::load(K, gi + a0 + x));
          vv = io<T>::load(V, gi + c0 + x);
        }
        sK[j][x] = (j0 + j < Ls) ? kv : 0.f;
        sV[j][x] = vv;
      }
      __syncthreads();
      const int jn = min(SW_KEYS, Ls - j0);
      for (int j = 0; j < jn; ++j) {
        const float k = sign * sK[j][ta];
        for (int c = 0; c < 4; ++c) acc[c] += k * sV[j][tc + c];
        if (z_lane) zacc += sign * sK[j][t];
      }
      __syncthreads();
    }
  }
  if (M_out) {
    for (int c = 0; c < 4; ++c) M_out[mbase + c] = acc[c];
    if (z_lane) z_out[bh * D + a0 + t] = zacc;
  }
}

template <typename T, int D>
static hipError_t sweep_t(const Geometry& g, const void* K, const void* V, const float* M_in,
                          const float* z_in, float* M_out, float* z_out, float* Msnap, float* zsnap,
                          int s_begin, int s_end, hipStream_t st, void* MsnapT, float sign) {
  dim3 grid((D / SW_TILE) * (D / SW_TILE), g.B * g.Hkv);
  hipLaunchKernelGGL((sweep_kernel<T, D>), grid, dim3(256), 0, st,
                     static_cast<const T*>(K), static_cast<const T*>(V), M_in, z_in, M_out, z_out,
                     Msnap, zsnap, static_cast<bf16_t*>(MsnapT), g.N, g.L, s_begin, s_end, g.lens, g.Hkv, sign);
  return hipGetLastError();
}

hipError_t launch_sweep(const Geometry& g, const void* K, const void* V, const float* M_in,
                        const float* z_in, float* M_out, float* z_out, float* Msnap, float* zsnap,
                        int s_begin, int s_end, hipStream_t st, void* MsnapT, bool subtract) {
  const float sign = subtract ? -1.f : 1.f;
#define SW_CASE(T, DD) return sweep_t<T, DD>(g, K, V, M_in, z_in, M_out, z_out, Msnap, zsnap, s_begin, s_end, st, MsnapT, sign)
  if (g.dtype == 0) {
    if (g.D == 32) SW_CASE(float, 32);
    if (g.D == 64) SW_CASE(float, 64);
    if (g.D == 128) SW_CASE(float, 128);
  } else {
    if (g.D == 32) SW_CASE(bf16_t, 32);
    if (g.D == 64) SW_CASE(bf16_t, 64);
    if (g.D == 128) SW_CASE(bf16_t, 128);
  }
#undef SW_CASE
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- generic forward

constexpr int GF_THREADS = 128;
constexpr int GF_KT = 32;        // keys per LDS tile

template <int D> struct RowSplit {
  static constexpr int LPR = D > 64 ? 2 : 1;      // lanes per query row
  static constexpr int DL = D / LPR;              // columns per lane
  static constexpr int ROWS = GF_THREADS / LPR;   // query rows per workgroup
};

template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (LPR >= 2) x += __shfl_xor(x, 1);
  if constexpr (LPR >= 4) x += __shfl_xor(x, 2);
  return x;
}

template <typename T, int D>
__global__ __launch_bounds__(GF_THREADS) void fwd_generic_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ beta, const float* __restrict__ Msnap, const float* __restrict__ zsnap,
    T* __restrict__ O, float* __restrict__ lse,
    int Hq, int Hkv, int N, int L, int s_begin, int nseg, float scale, const int* __restrict__ lens,
    const float* __restrict__ Amem) {
  using RS = RowSplit<D>;
  constexpr int LPR = RS::LPR, DL = RS::DL, ROWS = RS::ROWS;
  constexpr int LDS_FLOATS = (2 * GF_KT * D > D * D + D) ? 2 * GF_KT * D : D * D + D;
  __shared__ float smem[LDS_FLOATS];
  float* sK = smem;
  float* sV = smem + GF_KT * D;

  const int t = threadIdx.x;
  const int part = t % LPR;
  const int r = t / LPR;
  const int h = blockIdx.y;
  const int sl = blockIdx.z % nseg;
  const int b = blockIdx.z / nseg;
  const int s = s_begin + sl;
  const int kvh = h / (Hq / Hkv);
  // rows of this segment: the last may be short; none past the end of a
  // sequence of a variable-length batch
  const int Ls = min(L, seq_len_of(lens, b, N) - s * L);
  if (Ls <= 0) return;
  const int i_raw = blockIdx.x * ROWS + r;
  const bool valid = i_raw < Ls;
  const int i = valid ? i_raw : Ls - 1;
  const size_t qrow = (((size_t)b * Hq + h) * N + (size_t)s * L + i) * D + part * DL;
  const size_t kvbase = (((size_t)b * Hkv + kvh) * N + (size_t)s * L) * D;

  float q[DL], o[DL];
#pragma unroll
  for (int c = 0; c < DL; ++c) { q[c] = io<T>::load(Q, qrow + c) * scale; o[c] = 0.f; }
  float m = -INFINITY, l = 0.f;

  const int kend = min(Ls, (int)(blockIdx.x + 1) * ROWS);   // causal limit of this block
  for (int j0 = 0; j0 < kend; j0 += GF_KT) {
    for (int e = t; e < GF_KT * D; e += GF_THREADS) {
      const int j = e / D;
      const bool in = j0 + j < Ls;
      sK[e] = in ? io<T>::load(K, kvbase + (size_t)j0 * D + e) : 0.f;
      sV[e] = in ? io<T>::load(V, kvbase + (size_t)j0 * D + e) : 0.f;
    }
    __syncthreads();
    float sc[GF_KT];
    float mt = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < GF_KT; ++jj) {
      const float* kr = sK + jj * D + part * DL;
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < DL; ++c) acc += q[c] * kr[c];
      acc = row_sum<LPR>(acc);
      sc[jj] = (j0 + jj <= i) ? acc : -INFINITY;
      mt = fmaxf(mt, sc[jj]);
    }
    const float mn = fmaxf(m, mt);
    if (mn != -INFINITY) {
      const float corr = __expf(m - mn);
      l *= corr;
#pragma unroll
      for (int c = 0; c < DL; ++c) o[c] *= corr;
#pragma unroll
      for (int jj = 0; jj < GF_KT; ++jj) {
        const float p = __expf(sc[jj] - mn);
        l += p;
        const float* vr = sV + jj * D + part * DL;
#pragma unroll
        for (int c = 0; c < DL; ++c) o[c] += p * vr[c];
      }
      m = mn;
    }
    __syncthreads();
  }

  // Retrieval from M_{s-1}, z_{s-1} (or the A_mem rows formed by another
  // feature map's retrieval kernel) and the gate.
  float num[DL];
  float inv_den = 1.f;
  if (Amem) {
    const float* ar = Amem + (((size_t)b * Hq + h) * ((size_t)nseg * L) + (size_t)sl * L + i) * D + part * DL;
#pragma unroll
    for (int c = 0; c < DL; ++c) num[c] = ar[c];
  } else {
    const size_t snap = ((size_t)(b * Hkv + kvh) * nseg + sl);
    for (int e = t; e < D * D; e += GF_THREADS) smem[e] = Msnap[snap * D * D + e];
    for (int e = t; e < D; e += GF_THREADS) smem[D * D + e] = zsnap[snap * D + e];
    __syncthreads();
    const float* sM = smem;
    const float* sz = smem + D * D;
#pragma unroll
    for (int c = 0; c < DL; ++c) num[c] = 0.f;
    float den = 0.f;
    const size_t qfull = qrow - part * DL;
    for (int a = 0; a < D; ++a) {
      const float sq = elu1(io<T>::load(Q, qfull + a));
      den += sq * sz[a];
      const float* mr = sM + a * D + part * DL;
#pragma unroll
      for (int c = 0; c < DL; ++c) num[c] += sq * mr[c];
    }
    inv_den = 1.f / (den + 1e-6f);
  }
  const float gt = sigmoid(beta[h]);
  const float inv_l = 1.f / l;
  if (valid) {
#pragma unroll
    for (int c = 0; c < DL; ++c) {
      const float am = num[c] * inv_den;
      const float ad = o[c] * inv_l;
      io<T>::store(O, qrow + c, gt * am + (1.f - gt) * ad);
    }
    if (lse && part == 0) lse[((size_t)b * Hq + h) * N + (size_t)s * L + i] = m + __logf(l);
  }
}

template <typename T, int D>
static hipError_t fwd_t(const Geometry& g, const void* Q, const void* K, const void* V,
                        const float* beta, const float* Msnap, const float* zsnap, void* O,
                        float* lse, int s_begin, int s_end, hipStream_t st, const float* Amem) {
  using RS = RowSplit<D>;
  const int nseg = s_end - s_begin;
  dim3 grid((g.L + RS::ROWS - 1) / RS::ROWS, g.Hq, g.B * nseg);
  hipLaunchKernelGGL((fwd_generic_kernel<T, D>), grid, dim3(GF_THREADS), 0, st,
                     static_cast<const T*>(Q), static_cast<const T*>(K), static_cast<const T*>(V),
                     beta, Msnap, zsnap, static_cast<T*>(O), lse, g.Hq, g.Hkv, g.N, g.L, s_begin,
                     nseg, 1.f / sqrtf((float)D), g.lens, Amem);
  return hipGetLastError();
}

hipError_t launch_fwd_generic(const Geometry& g, const void* Q, const void* K, const void* V,
                              const float* beta, const float* Msnap, const float* zsnap, void* O,
                              float* lse, int s_begin, int s_end, hipStream_t st, const float* Amem) {
#define GF_CASE(T, DD) return fwd_t<T, DD>(g, Q, K, V, beta, Msnap, zsnap, O, lse, s_begin, s_end, st, Amem)
  if (g.dtype == 0) {
    if (g.D == 32) GF_CASE(float, 32);
    if (g.D == 64) GF_CASE(float, 64);
    if (g.D == 128) GF_CASE(float, 128);
  } else {
    if (g.D == 32) GF_CASE(bf16_t, 32);
    if (g.D == 64) GF_CASE(bf16_t, 64);
    if (g.D == 128) GF_CASE(bf16_t, 128);
  }
#undef GF_CASE
  return hipErrorInvalidValue;
}

// dst[i] = src ? src[i] : 0 for i < n (the state an empty sequence passes
// through unchanged, or its gradient).
__global__ __launch_bounds__(256) void state_copy_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                         size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_state_copy(float* dst, const float* src, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st, dst, src, n);
  return hipGetLastError();
}

// Rows [n_b, N) of slot (b, h): one workgroup per (b, h), 32-bit stores.
__global__ __launch_bounds__(256) void zero_tail_kernel(uint32_t* __restrict__ X, const int* __restrict__ lens,
                                                       int H, int N, size_t row_words) {
  const int bh = blockIdx.x;
  const int nb = seq_len_of(lens, bh / H, N);
  uint32_t* base = X + (size_t)bh * N * row_words;
  const size_t first = (size_t)nb * row_words, end = (size_t)N * row_words;
  for (size_t i = first + threadIdx.x; i < end; i += 256) base[i] = 0u;
}

hipError_t launch_zero_tail(void* X, const int* lens, int B, int H, int N, size_t row_words, hipStream_t st) {
  if (!X || !lens || (long long)B * H == 0 || N == 0) return hipSuccess;
  if ((long long)B * H > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(zero_tail_kernel, dim3((unsigned)(B * H)), dim3(256), 0, st, static_cast<uint32_t*>(X), lens,
                     H, N, row_words);
  return hipGetLastError();
}

}  // namespace infini
