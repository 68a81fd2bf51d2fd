// Generic backward of the Infini-attention segment kernel (fp32 vector ALU).
//
// The pages give only the forward (page "Hugging Face Infini-Attention 재현
// 분석", section "Infini-Attention 메커니즘"); this is its exact derivative.
// With g = sigmoid(beta), dA_mem = g dO and dA_dot = (1 - g) dO:
//   gate:       dbeta = g (1 - g) sum dO * (A_mem - A_dot), both terms recomputed
//               in fp32 (never recovered from the rounded output)
//   retrieval:  dnum = dA_mem / den, dden = -rowsum(dA_mem * A_mem) / den,
//               dQ += (dnum M_{s-1}^T + dden z_{s-1}^T) * sigma'(Q),
//               and dL/dM_{s-1} gains sigma(Q)^T dnum, dL/dz_{s-1} gains sigma(Q)^T dden
//   local:      P recomputed from the row log-sum-exp, D_i = rowsum(dA_dot * A_dot),
//               dS = P * (dA_dot V^T - D_i), dQ += dS K / sqrt d,
//               dK += dS^T Q / sqrt d, dV += P^T dA_dot
//   update:     with dM = dL/dM_s, dV += sigma(K) dM,
//               dK += (V dM^T + 1 dz^T) * sigma'(K)
// dL/dM_s is a suffix sum over later segments of the retrieval terms; it is
// formed by `rscan_kernel`, the reverse counterpart of the forward sweep, so
// that every segment's backward runs in parallel.
#include "common.h"
#include "kernels.h"

namespace infini {

constexpr int GB_THREADS = 128;
constexpr int GB_KT = 32;      // keys per LDS tile (query-side kernel)
constexpr int GB_QT = 16;      // query rows per LDS tile (key-side kernel)

template <int LPR>
__device__ __forceinline__ float lanes_sum(float x) {
  if constexpr (LPR >= 2) x += __shfl_xor(x, 1);
  if constexpr (LPR >= 4) x += __shfl_xor(x, 2);
  return x;
}

template <int D> struct QSplit {
  static constexpr int LPR = D / 32;          // 32 columns per lane keeps register arrays small
  static constexpr int DL = 32;
  static constexpr int ROWS = GB_THREADS / LPR;
};
template <int D> struct KSplit {
  static constexpr int LPR = D / 32;          // 32 columns per lane
  static constexpr int DL = 32;
  static constexpr int ROWS = GB_THREADS / LPR;
};

int bwd_q_row_blocks(const Geometry& g) {
  if (bwd_long_mfma_supported(g)) return bwd_q_mfma_row_blocks(g);
  const int rows = GB_THREADS / (g.D / 32);
  return (g.L + rows - 1) / rows;
}

// ---------------------------------------------------------------- query side

template <typename T, int D>
__global__ __launch_bounds__(GB_THREADS) void bwd_q_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ beta, const float* __restrict__ Msnap, const float* __restrict__ zsnap,
    const T* __restrict__ dO, T* __restrict__ dQ,
    float* __restrict__ ws_lse, float* __restrict__ ws_Dd, float* __restrict__ ws_dden,
    float* __restrict__ ws_dnum, float* __restrict__ dbeta_part, const float* __restrict__ lse_in,
    int Hq, int Hkv, int N, int L, int s_begin, int nseg, float scale, const int* __restrict__ lens) {
  using RS = QSplit<D>;
  constexpr int LPR = RS::LPR, DL = RS::DL, ROWS = RS::ROWS;
  constexpr int REGION_A = (2 * GB_KT * D > D * D + D) ? 2 * GB_KT * D : D * D + D;
  constexpr int RSTRIDE = D + 1;
  __shared__ float smem[REGION_A + ROWS * RSTRIDE + GB_THREADS];
  float* sK = smem;
  float* sV = smem + GB_KT * D;
  float* srow = smem + REGION_A;                   // per-row dnum
  float* sred = srow + ROWS * RSTRIDE;             // dbeta block reduction

  const int t = threadIdx.x;
  const int part = t % LPR;
  const int r = t / LPR;
  const int h = blockIdx.y;
  const int sl = blockIdx.z % nseg;
  const int b = blockIdx.z / nseg;
  const int s = s_begin + sl;
  const int kvh = h / (Hq / Hkv);
  // rows of this segment: the last may be short; none past the end of a
  // sequence of a variable-length batch (its dbeta part is then zero)
  const int Ls = min(L, seq_len_of(lens, b, N) - s * L);
  if (Ls <= 0) {
    if (t == 0) dbeta_part[(((size_t)b * Hq + h) * nseg + sl) * gridDim.x + blockIdx.x] = 0.f;
    return;
  }
  const int i_raw = blockIdx.x * ROWS + r;
  const bool valid = i_raw < Ls;
  const int i = valid ? i_raw : Ls - 1;
  const size_t qrow = (((size_t)b * Hq + h) * N + (size_t)s * L + i) * D + part * DL;
  const size_t kvbase = (((size_t)b * Hkv + kvh) * N + (size_t)s * L) * D;
  const size_t crow = ((size_t)b * Hq + h) * ((size_t)nseg * L) + (size_t)sl * L + i;  // chunk row

  float q[DL], o[DL];
#pragma unroll
  for (int c = 0; c < DL; ++c) { q[c] = io<T>::load(Q, qrow + c); o[c] = 0.f; }
  // With the forward's row log-sum-exp the probabilities are final as they
  // are formed (m = lse, l = 1, no rescale); otherwise the running max and
  // sum are kept as usual.
  const float lse_row = lse_in ? lse_in[((size_t)b * Hq + h) * N + (size_t)s * L + i] : 0.f;
  float m = lse_in ? lse_row : -INFINITY, l = lse_in ? 1.f : 0.f;
  const int kend = min(Ls, (int)(blockIdx.x + 1) * ROWS);

  // Pass 1: recompute A_dot and the row log-sum-exp.
  for (int j0 = 0; j0 < kend; j0 += GB_KT) {
    for (int e = t; e < GB_KT * D; e += GB_THREADS) {
      const bool in = j0 + e / D < Ls;
      sK[e] = in ? io<T>::load(K, kvbase + (size_t)j0 * D + e) : 0.f;
      sV[e] = in ? io<T>::load(V, kvbase + (size_t)j0 * D + e) : 0.f;
    }
    __syncthreads();
    float sc[GB_KT];
    float mt = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < GB_KT; ++jj) {
      const float* kr = sK + jj * D + part * DL;
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < DL; ++c) acc += q[c] * kr[c];
      acc = lanes_sum<LPR>(acc) * scale;
      sc[jj] = (j0 + jj <= i) ? acc : -INFINITY;
      mt = fmaxf(mt, sc[jj]);
    }
    const float mn = lse_in ? m : fmaxf(m, mt);
    if (!lse_in) {
      const float corr = __expf(m - mn);
      l *= corr;
#pragma unroll
      for (int c = 0; c < DL; ++c) o[c] *= corr;
    }
#pragma unroll
    for (int jj = 0; jj < GB_KT; ++jj) {
      const float p = __expf(sc[jj] - mn);
      if (!lse_in) l += p;
      const float* vr = sV + jj * D + part * DL;
#pragma unroll
      for (int c = 0; c < DL; ++c) o[c] += p * vr[c];
    }
    m = mn;
    __syncthreads();
  }
  const float lse = lse_in ? lse_row : m + __logf(l);
  const float inv_l = 1.f / l;
  const float gt = sigmoid(beta[h]);
  const float og = 1.f - gt;
  // A_dot, then dA_dot = (1 - g) dO in place; t1 = sum dO * A_dot.
  float t1 = 0.f;
#pragma unroll
  for (int c = 0; c < DL; ++c) {
    const float g_o = io<T>::load(dO, qrow + c);
    t1 += g_o * (o[c] * inv_l);
    o[c] = og * g_o;
  }
  t1 = lanes_sum<LPR>(t1);
  const float Dd = og * t1;                             // rowsum(dA_dot * A_dot)

  // Pass 2: dQ_local = sum_j P_ij (dP_ij - D_i) k_j  (scale applied at the end).
  float dql[DL];
#pragma unroll
  for (int c = 0; c < DL; ++c) dql[c] = 0.f;
  for (int j0 = 0; j0 < kend; j0 += GB_KT) {
    for (int e = t; e < GB_KT * D; e += GB_THREADS) {
      const bool in = j0 + e / D < Ls;
      sK[e] = in ? io<T>::load(K, kvbase + (size_t)j0 * D + e) : 0.f;
      sV[e] = in ? io<T>::load(V, kvbase + (size_t)j0 * D + e) : 0.f;
    }
    __syncthreads();
    for (int jj = 0; jj < GB_KT; ++jj) {
      const float* kr = sK + jj * D + part * DL;
      const float* vr = sV + jj * D + part * DL;
      float sdot = 0.f, pdot = 0.f;
#pragma unroll
      for (int c = 0; c < DL; ++c) { sdot += q[c] * kr[c]; pdot += o[c] * vr[c]; }
      sdot = lanes_sum<LPR>(sdot) * scale;
      pdot = lanes_sum<LPR>(pdot);
      const float p = (j0 + jj <= i) ? __expf(sdot - lse) : 0.f;
      const float ds = p * (pdot - Dd);
#pragma unroll
      for (int c = 0; c < DL; ++c) dql[c] += ds * kr[c];
    }
    __syncthreads();
  }

  // Retrieval recompute from M_{s-1}, z_{s-1}.
  const size_t snap = ((size_t)(b * Hkv + kvh) * nseg + sl);
  for (int e = t; e < D * D; e += GB_THREADS) smem[e] = Msnap[snap * D * D + e];
  for (int e = t; e < D; e += GB_THREADS) smem[D * D + e] = zsnap[snap * D + e];
  __syncthreads();
  const float* sM = smem;
  const float* sz = smem + D * D;
  float num[DL];
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
  den += 1e-6f;
  const float inv_den = 1.f / den;
  // t2 = sum dO * A_mem; dnum = g dO / den; dden = -g t2 / den.
  float t2 = 0.f;
#pragma unroll
  for (int c = 0; c < DL; ++c) {
    const float g_o = io<T>::load(dO, qrow + c);
    t2 += g_o * (num[c] * inv_den);
    num[c] = gt * g_o * inv_den;
  }
  t2 = lanes_sum<LPR>(t2);
  const float dd = -gt * t2 * inv_den;
  const float bsum = valid ? t2 - t1 : 0.f;
#pragma unroll
  for (int c = 0; c < DL; ++c) srow[r * RSTRIDE + part * DL + c] = num[c];
  if (part == 0) sred[r] = bsum;
  if (valid) {
#pragma unroll
    for (int c = 0; c < DL; ++c) ws_dnum[crow * D + part * DL + c] = num[c];
    if (part == 0) { ws_lse[crow] = lse; ws_Dd[crow] = Dd; ws_dden[crow] = dd; }
  }
  __syncthreads();
  // dsigma(Q)_a = sum_c dnum_c M[a][c] + dden z_a, for this lane's columns a.
  float dsq[DL];
#pragma unroll
  for (int x = 0; x < DL; ++x) dsq[x] = dd * sz[part * DL + x];
  for (int c = 0; c < D; ++c) {
    const float dn = srow[r * RSTRIDE + c];
    const float* mc = sM + (size_t)part * DL * D + c;
#pragma unroll
    for (int x = 0; x < DL; ++x) dsq[x] += dn * mc[x * D];
  }
  if (t == 0) {
    float tot = 0.f;
    for (int x = 0; x < ROWS; ++x) tot += sred[x];
    dbeta_part[(((size_t)b * Hq + h) * nseg + sl) * gridDim.x + blockIdx.x] = tot;
  }
  if (valid) {
#pragma unroll
    for (int c = 0; c < DL; ++c)
      io<T>::store(dQ, qrow + c, dsq[c] * elu1_grad(q[c]) + scale * dql[c]);
  }
}

template <typename T, int D>
static hipError_t bwd_q_t(const Geometry& g, const void* Q, const void* K, const void* V,
                          const float* beta, const float* Msnap, const float* zsnap, const void* dO,
                          void* dQ, const BwdChunkWs& w, const float* lse_in, int s_begin, int s_end,
                          hipStream_t st) {
  using RS = QSplit<D>;
  const int nseg = s_end - s_begin;
  dim3 grid((g.L + RS::ROWS - 1) / RS::ROWS, g.Hq, g.B * nseg);
  hipLaunchKernelGGL((bwd_q_kernel<T, D>), grid, dim3(GB_THREADS), 0, st,
                     static_cast<const T*>(Q), static_cast<const T*>(K), static_cast<const T*>(V),
                     beta, Msnap, zsnap, static_cast<const T*>(dO), static_cast<T*>(dQ), w.lse, w.Dd,
                     w.dden, w.dnum, w.dbeta_part, lse_in, g.Hq, g.Hkv, g.N, g.L, s_begin, nseg,
                     1.f / sqrtf((float)D), g.lens);
  return hipGetLastError();
}

// ---------------------------------------------------------------- reverse state scan

constexpr int RS_TILE = 32;
constexpr int RS_ROWS = 64;

template <typename T, int D>
__global__ __launch_bounds__(256) void rscan_kernel(
    const T* __restrict__ Q, const float* __restrict__ dnum, const float* __restrict__ dden,
    const float* dM_in, const float* dz_in, float* dM_out, float* dz_out,
    float* __restrict__ dMsnap, float* __restrict__ dzsnap,
    int Hq, int Hkv, int N, int L, int s_begin, int nseg, const int* __restrict__ lens) {
  constexpr int TPR = D / RS_TILE;
  const int tile = blockIdx.x;
  const int a0 = (tile / TPR) * RS_TILE;
  const int c0 = (tile % TPR) * RS_TILE;
  const bool do_z = (tile % TPR) == 0;
  const int bk = blockIdx.y;
  const int b = bk / Hkv, kvh = bk % Hkv;
  const int G = Hq / Hkv;
  const int t = threadIdx.x;
  const int ta = t >> 3;
  const int tc = (t & 7) * 4;
  const bool z_lane = do_z && t < RS_TILE;

  __shared__ float sQ[RS_ROWS][RS_TILE + 1];
  __shared__ float sN[RS_ROWS][RS_TILE + 4];
  __shared__ float sD[RS_ROWS];

  float acc[4];
  float zacc = 0.f;
  const size_t mbase = (size_t)bk * D * D + (size_t)(a0 + ta) * D + c0 + tc;
  for (int c = 0; c < 4; ++c) acc[c] = dM_in ? dM_in[mbase + c] : 0.f;
  if (z_lane) zacc = dz_in ? dz_in[(size_t)bk * D + a0 + t] : 0.f;

  for (int sl = nseg - 1; sl >= 0; --sl) {
    const int s = s_begin + sl;
    const size_t sb = ((size_t)bk * nseg + sl) * D * D + (size_t)(a0 + ta) * D + c0 + tc;
    for (int c = 0; c < 4; ++c) dMsnap[sb + c] = acc[c];
    if (z_lane) dzsnap[((size_t)bk * nseg + sl) * D + a0 + t] = zacc;
    // rows of this segment (the last may be short; none past a sequence's end)
    const int Ls = min(L, seq_len_of(lens, b, N) - s * L);
    for (int h = kvh * G; h < (kvh + 1) * G; ++h) {
      const size_t qbase = (((size_t)b * Hq + h) * N + (size_t)s * L) * D;
      const size_t cbase = ((size_t)b * Hq + h) * ((size_t)nseg * L) + (size_t)sl * L;
      for (int i0 = 0; i0 < Ls; i0 += RS_ROWS) {
        for (int e = t; e < RS_ROWS * RS_TILE; e += 256) {
          const int i = e / RS_TILE, x = e % RS_TILE;
          const bool in = i0 + i < Ls;
          sQ[i][x] = in ? elu1(io<T>::load(Q, qbase + (size_t)(i0 + i) * D + a0 + x)) : 0.f;
          sN[i][x] = in ? dnum[(cbase + i0 + i) * D + c0 + x] : 0.f;
        }
        for (int e = t; e < RS_ROWS; e += 256) sD[e] = (i0 + e < Ls) ? dden[cbase + i0 + e] : 0.f;
        __syncthreads();
        const int in_n = min(RS_ROWS, Ls - i0);
        for (int i = 0; i < in_n; ++i) {
          const float sq = sQ[i][ta];
          for (int c = 0; c < 4; ++c) acc[c] += sq * sN[i][tc + c];
          if (z_lane) zacc += sQ[i][t] * sD[i];
        }
        __syncthreads();
      }
    }
  }
  if (dM_out) {
    for (int c = 0; c < 4; ++c) dM_out[mbase + c] = acc[c];
    if (z_lane) dz_out[(size_t)bk * D + a0 + t] = zacc;
  }
}

template <typename T, int D>
static hipError_t rscan_t(const Geometry& g, const void* Q, const BwdChunkWs& w, const float* dM_in,
                          const float* dz_in, float* dM_out, float* dz_out, int s_begin, int s_end,
                          hipStream_t st) {
  dim3 grid((D / RS_TILE) * (D / RS_TILE), g.B * g.Hkv);
  hipLaunchKernelGGL((rscan_kernel<T, D>), grid, dim3(256), 0, st, static_cast<const T*>(Q), w.dnum,
                     w.dden, dM_in, dz_in, dM_out, dz_out, w.dMsnap, w.dzsnap, g.Hq, g.Hkv, g.N,
                     g.L, s_begin, s_end - s_begin, g.lens);
  return hipGetLastError();
}

// ---------------------------------------------------------------- key side

template <typename T, int D>
__global__ __launch_bounds__(GB_THREADS) void bwd_kv_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ beta, const T* __restrict__ dO,
    const float* __restrict__ ws_lse, const float* __restrict__ ws_Dd,
    const float* __restrict__ dMsnap, const float* __restrict__ dzsnap,
    T* __restrict__ dK, T* __restrict__ dV,
    int Hq, int Hkv, int N, int L, int s_begin, int nseg, float scale, const int* __restrict__ lens) {
  using RS = KSplit<D>;
  constexpr int LPR = RS::LPR, DL = RS::DL, ROWS = RS::ROWS;
  constexpr int RST = D + 1;
  constexpr int REGION_A = (2 * GB_QT * D + 2 * GB_QT > D * D + D) ? 2 * GB_QT * D + 2 * GB_QT : D * D + D;
  __shared__ float smem[REGION_A + 2 * ROWS * RST];
  float* sQ = smem;
  float* sO = smem + GB_QT * D;
  float* sL = smem + 2 * GB_QT * D;
  float* sDd = sL + GB_QT;
  float* skrow = smem + REGION_A;              // sigma(k_j) rows
  float* svrow = skrow + ROWS * RST;           // v_j rows

  const int t = threadIdx.x;
  const int part = t % LPR;
  const int r = t / LPR;
  const int kvh = blockIdx.y;
  const int sl = blockIdx.z % nseg;
  const int b = blockIdx.z / nseg;
  const int s = s_begin + sl;
  const int G = Hq / Hkv;
  // keys of this segment: the last may be short; none past the end of a
  // sequence of a variable-length batch
  const int Ls = min(L, seq_len_of(lens, b, N) - s * L);
  if (Ls <= 0) return;
  const int j_raw = blockIdx.x * ROWS + r;
  const bool valid = j_raw < Ls;
  const int j = valid ? j_raw : Ls - 1;
  const size_t krow = (((size_t)b * Hkv + kvh) * N + (size_t)s * L + j) * D + part * DL;

  float k[DL], v[DL], dk[DL], dv[DL];
#pragma unroll
  for (int c = 0; c < DL; ++c) {
    k[c] = io<T>::load(K, krow + c);
    v[c] = io<T>::load(V, krow + c);
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  const int i_start = blockIdx.x * ROWS;      // first query row that can see this block's keys

  for (int h = kvh * G; h < (kvh + 1) * G; ++h) {
    const float gt = sigmoid(beta[h]);
    const float og = 1.f - gt;
    const size_t qbase = (((size_t)b * Hq + h) * N + (size_t)s * L) * D;
    const size_t cbase = ((size_t)b * Hq + h) * ((size_t)nseg * L) + (size_t)sl * L;
    for (int i0 = i_start; i0 < Ls; i0 += GB_QT) {
      for (int e = t; e < GB_QT * D; e += GB_THREADS) {
        const bool in = i0 + e / D < Ls;
        sQ[e] = in ? io<T>::load(Q, qbase + (size_t)i0 * D + e) : 0.f;
        sO[e] = in ? io<T>::load(dO, qbase + (size_t)i0 * D + e) : 0.f;
      }
      for (int e = t; e < GB_QT; e += GB_THREADS) {
        const bool in = i0 + e < Ls;
        sL[e] = in ? ws_lse[cbase + i0 + e] : 0.f;
        sDd[e] = in ? ws_Dd[cbase + i0 + e] : 0.f;
      }
      __syncthreads();
      const int qn = min(GB_QT, Ls - i0);
      for (int ii = 0; ii < qn; ++ii) {
        const float* qr = sQ + ii * D + part * DL;
        const float* orow = sO + ii * D + part * DL;
        float sdot = 0.f, pdot = 0.f;
#pragma unroll
        for (int c = 0; c < DL; ++c) { sdot += qr[c] * k[c]; pdot += orow[c] * v[c]; }
        sdot = lanes_sum<LPR>(sdot) * scale;
        pdot = lanes_sum<LPR>(pdot) * og;
        const float p = (i0 + ii >= j) ? __expf(sdot - sL[ii]) : 0.f;
        const float ds = p * (pdot - sDd[ii]);
        const float pg = p * og;
#pragma unroll
        for (int c = 0; c < DL; ++c) {
          dv[c] += pg * orow[c];
          dk[c] += ds * qr[c];
        }
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int c = 0; c < DL; ++c) dk[c] *= scale;

  // Update backward with dM = dL/dM_s.
  const size_t snap = ((size_t)(b * Hkv + kvh) * nseg + sl);
  for (int e = t; e < D * D; e += GB_THREADS) smem[e] = dMsnap[snap * D * D + e];
  for (int e = t; e < D; e += GB_THREADS) smem[D * D + e] = dzsnap[snap * D + e];
#pragma unroll
  for (int c = 0; c < DL; ++c) {
    skrow[r * RST + part * DL + c] = elu1(k[c]);
    svrow[r * RST + part * DL + c] = v[c];
  }
  __syncthreads();
  const float* sM = smem;
  const float* sz = smem + D * D;
  // dsigma(k)_a = sum_c v_c dM[a][c] + dz_a for this lane's a; dv_c += sum_a sigma(k)_a dM[a][c].
  float dsk[DL];
#pragma unroll
  for (int x = 0; x < DL; ++x) dsk[x] = sz[part * DL + x];
  for (int c = 0; c < D; ++c) {
    const float vc = svrow[r * RST + c];
    const float* mc = sM + (size_t)part * DL * D + c;
#pragma unroll
    for (int x = 0; x < DL; ++x) dsk[x] += vc * mc[x * D];
  }
#pragma unroll
  for (int x = 0; x < DL; ++x) dk[x] += dsk[x] * elu1_grad(k[x]);
  for (int a = 0; a < D; ++a) {
    const float sk = skrow[r * RST + a];
    const float* mr = sM + a * D + part * DL;
#pragma unroll
    for (int c = 0; c < DL; ++c) dv[c] += sk * mr[c];
  }
  if (valid) {
#pragma unroll
    for (int c = 0; c < DL; ++c) {
      io<T>::store(dK, krow + c, dk[c]);
      io<T>::store(dV, krow + c, dv[c]);
    }
  }
}

template <typename T, int D>
static hipError_t bwd_kv_t(const Geometry& g, const void* Q, const void* K, const void* V,
                           const float* beta, const void* dO, const BwdChunkWs& w, void* dK, void* dV,
                           int s_begin, int s_end, hipStream_t st) {
  using RS = KSplit<D>;
  const int nseg = s_end - s_begin;
  dim3 grid((g.L + RS::ROWS - 1) / RS::ROWS, g.Hkv, g.B * nseg);
  hipLaunchKernelGGL((bwd_kv_kernel<T, D>), grid, dim3(GB_THREADS), 0, st,
                     static_cast<const T*>(Q), static_cast<const T*>(K), static_cast<const T*>(V),
                     beta, static_cast<const T*>(dO), w.lse, w.Dd, w.dMsnap, w.dzsnap,
                     static_cast<T*>(dK), static_cast<T*>(dV), g.Hq, g.Hkv, g.N, g.L, s_begin, nseg,
                     1.f / sqrtf((float)D), g.lens);
  return hipGetLastError();
}

// ---------------------------------------------------------------- dbeta

__global__ void dbeta_reduce_kernel(const float* __restrict__ beta, const float* __restrict__ part,
                                    float* dbeta_acc, float* dbeta, int B, int Hq, int nseg,
                                    int nblk, int first, int last) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= Hq) return;
  float tot = first ? 0.f : dbeta_acc[h];
  for (int b = 0; b < B; ++b)
    for (int x = 0; x < nseg * nblk; ++x) tot += part[((size_t)b * Hq + h) * nseg * nblk + x];
  dbeta_acc[h] = tot;
  if (last) {
    const float gt = sigmoid(beta[h]);
    dbeta[h] = gt * (1.f - gt) * tot;
  }
}

hipError_t launch_dbeta_reduce(const Geometry& g, const float* beta, const BwdChunkWs& w,
                               float* dbeta_acc, float* dbeta, int nseg, bool first, bool last,
                               hipStream_t st) {
  hipLaunchKernelGGL(dbeta_reduce_kernel, dim3((g.Hq + 63) / 64), dim3(64), 0, st, beta,
                     w.dbeta_part, dbeta_acc, dbeta, g.B, g.Hq, nseg, bwd_q_row_blocks(g),
                     first ? 1 : 0, last ? 1 : 0);
  return hipGetLastError();
}

// ---------------------------------------------------------------- dispatch

#define DISPATCH_TD(FN, ...)                                        \
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

hipError_t launch_bwd_q(const Geometry& g, const void* Q, const void* K, const void* V,
                        const float* beta, const float* Msnap, const float* zsnap, const void* dO,
                        void* dQ, const BwdChunkWs& w, const float* lse_in, int s_begin, int s_end,
                        hipStream_t st) {
  DISPATCH_TD(bwd_q_t, g, Q, K, V, beta, Msnap, zsnap, dO, dQ, w, lse_in, s_begin, s_end, st);
}

hipError_t launch_rscan(const Geometry& g, const void* Q, const BwdChunkWs& w, const float* dM_in,
                        const float* dz_in, float* dM_out, float* dz_out, int s_begin, int s_end,
                        hipStream_t st) {
  DISPATCH_TD(rscan_t, g, Q, w, dM_in, dz_in, dM_out, dz_out, s_begin, s_end, st);
}

hipError_t launch_bwd_kv(const Geometry& g, const void* Q, const void* K, const void* V,
                         const float* beta, const void* dO, const BwdChunkWs& w, void* dK, void* dV,
                         int s_begin, int s_end, hipStream_t st) {
  if (bwd_long_mfma_supported(g)) return launch_bwd_kv_mfma(g, Q, K, V, beta, dO, w, dK, dV, s_begin, s_end, st);
  DISPATCH_TD(bwd_kv_t, g, Q, K, V, beta, dO, w, dK, dV, s_begin, s_end, st);
}

}  // namespace infini
