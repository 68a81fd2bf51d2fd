// Streaming decode: new tokens appended to the segment that is being filled.
//
// The forward of a whole segment (page "Hugging Face Infini-Attention 재현
// 분석", section "Infini-Attention 메커니즘": Local Attention, Memory
// Retrieval, Integration) evaluated for a few rows at a time: row i of the
// current segment attends causally to the segment's keys 0..i, of which rows
// 0..pos-1 are already in the caller's K/V cache and rows pos.. arrive with
// this call; retrieval reads the state before the segment.  The memory update
// (Memory Update) runs once the segment is full, over the cache, with the
// ordinary memory-phase kernels.
//
// One workgroup per (batch, K/V head, key split) serves the group's query
// heads and the call's new rows one after another.  With few (batch, K/V
// head) pairs the keys of each row are split over several workgroups so that
// the whole chip reads the cache; each writes its partial softmax state
// (max, sum, unnormalised P V row) and decode_combine_kernel merges the parts
// by the same identity, then adds retrieval and the gate.  Per row: scores of up to DC_CHUNK keys
// at a time (one key per thread, the query in LDS), the chunk's softmax merged
// into the running (max, sum) by the online-softmax identity (page "Context
// Memorization for Efficient Long Context Generation", section "방법론"), and
// P V with one 16-byte column chunk per thread and the keys split over the
// remaining thread groups.  Decode is bound by reading the cached K and V
// once per row.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace infini {

constexpr int DC_THREADS = 256;
constexpr int DC_CHUNK = 1024;                 // keys scored per pass (4 per thread)
constexpr int PB = 4;                          // V rows per thread in flight in the P V pass

template <typename T> struct vec16;            // one 16-byte load, then as floats
template <> struct vec16<float> {
  static constexpr int N = 4;
  using R = float4;
  __device__ __forceinline__ static R raw(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ static void cvt(const R& v, float (&x)[4]) {
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
  __device__ __forceinline__ static void load(const float* p, float (&x)[4]) { cvt(raw(p), x); }
};
template <> struct vec16<bf16_t> {
  static constexpr int N = 8;
  using R = uint4;
  __device__ __forceinline__ static R raw(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ static void cvt(const R& v, float (&x)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void load(const bf16_t* p, float (&x)[8]) { cvt(raw(p), x); }
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_add(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <typename T, int D>
__global__ __launch_bounds__(DC_THREADS) void decode_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ beta, T* __restrict__ Kc, T* __restrict__ Vc,
    const float* __restrict__ M, const float* __restrict__ z, T* __restrict__ O,
    float* __restrict__ part, int Hq, int Hkv, int Tn, int L, int pos, int nsplit, int split_keys,
    float scale) {
  constexpr int VW = vec16<T>::N;              // elements per 16-byte load
  constexpr int NCH = D / VW;                  // 16-byte chunks per row
  constexpr int NKG = DC_THREADS / NCH;        // key groups in the P V pass
  __shared__ float sp[DC_CHUNK];               // scores, then probabilities, of a chunk
  __shared__ float sq[D];                      // the query row
  __shared__ float sred[2][DC_THREADS / 64];
  __shared__ float so[NKG][D + 1];

  const int bk = blockIdx.x / nsplit, sp_id = blockIdx.x % nsplit;
  const int b = bk / Hkv, kvh = bk % Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int ch = tid % NCH, kgp = tid / NCH;  // P V: columns ch*VW .. +VW-1, keys kgp + NKG*n
  const size_t cbase = (size_t)bk * L * D;     // cache rows of this (batch, K/V head)
  const size_t nbase = (size_t)bk * Tn * D;    // this call's new K/V rows

  // Append the new rows to the cache (split 0).  The scores below read new
  // keys from K and V themselves, so nothing waits for these stores.
  for (int e = tid; sp_id == 0 && e < Tn * D; e += DC_THREADS) {
    Kc[cbase + (size_t)pos * D + e] = K[nbase + e];
    Vc[cbase + (size_t)pos * D + e] = V[nbase + e];
  }
  auto krow = [&](int j) { return j < pos ? Kc + cbase + (size_t)j * D : K + nbase + (size_t)(j - pos) * D; };
  auto vrow = [&](int j) { return j < pos ? Vc + cbase + (size_t)j * D : V + nbase + (size_t)(j - pos) * D; };

  for (int h = kvh * G; h < (kvh + 1) * G; ++h) {
    const float gt = sigmoid(beta[h]);
    for (int t = 0; t < Tn; ++t) {
      const int i = pos + t;                   // row inside the segment
      const size_t qrow = (((size_t)b * Hq + h) * Tn + t) * D;
      // every thread holds the query row itself, so the key loads below do
      // not wait for a barrier; sq (read by the retrieval, after the chunk
      // loop's barriers) is written beside it
      float qv[D];
#pragma unroll
      for (int a0 = 0; a0 < D; a0 += VW) {
        float x[VW];
        vec16<T>::load(Q + qrow + a0, x);
#pragma unroll
        for (int e = 0; e < VW; ++e) qv[a0 + e] = x[e];
      }
      for (int a = tid; a < D; a += DC_THREADS) sq[a] = io<T>::load(Q, qrow + a);

      float m = -INFINITY, l = 0.f;
      float oc[VW];
#pragma unroll
      for (int e = 0; e < VW; ++e) oc[e] = 0.f;
      const int klo = sp_id * split_keys;      // this split's keys of row i: [klo, khi)
      const int khi = min(klo + split_keys, i + 1);
      for (int j0 = klo; j0 < khi; j0 += DC_CHUNK) {
        const int jn = min(DC_CHUNK, khi - j0);
        float cm = -INFINITY;
#pragma unroll
        for (int r = 0; r < DC_CHUNK / DC_THREADS; ++r) {
          const int jj = tid + DC_THREADS * r;
          float s = -INFINITY;
          if (jj < jn) {
            const T* kr = krow(j0 + jj);
            float acc = 0.f;
#pragma unroll
            for (int a0 = 0; a0 < D; a0 += VW) {
              float x[VW];
              vec16<T>::load(kr + a0, x);
#pragma unroll
              for (int e = 0; e < VW; ++e) acc = fmaf(qv[a0 + e], x[e], acc);
            }
            s = acc * scale;
          }
          sp[jj] = s;
          cm = fmaxf(cm, s);
        }
        // the first P V batch of V rows is loaded while the scores reduce
        // (indexes past the chunk repeat its last key and get weight 0)
        typename vec16<T>::R vr[PB];
#pragma unroll
        for (int u = 0; u < PB; ++u) vr[u] = vec16<T>::raw(vrow(j0 + min(kgp + NKG * u, jn - 1)) + ch * VW);
        cm = wave_max(cm);
        if ((tid & 63) == 0) sred[0][wave] = cm;
        __syncthreads();
        cm = sred[0][0];
#pragma unroll
        for (int w = 1; w < DC_THREADS / 64; ++w) cm = fmaxf(cm, sred[0][w]);
        const float mn = fmaxf(m, cm);         // finite: every chunk holds at least one key
        const float corr = __expf(m - mn);
#pragma unroll
        for (int e = 0; e < VW; ++e) oc[e] *= corr;
        l *= corr;
        m = mn;
        float lp = 0.f;
#pragma unroll
        for (int r = 0; r < DC_CHUNK / DC_THREADS; ++r) {
          const int jj = tid + DC_THREADS * r;
          if (jj < jn) {
            const float p = __expf(sp[jj] - m);
            sp[jj] = p;
            lp += p;
          }
        }
        lp = wave_add(lp);
        if ((tid & 63) == 0) sred[1][wave] = lp;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < DC_THREADS / 64; ++w) l += sred[1][w];
        for (int jb = kgp; jb < jn; jb += NKG * PB) {
          const bool more = jb + NKG * PB < jn;
          typename vec16<T>::R nx[PB];
          if (more) {
#pragma unroll
            for (int u = 0; u < PB; ++u)
              nx[u] = vec16<T>::raw(vrow(j0 + min(jb + NKG * (PB + u), jn - 1)) + ch * VW);
          }
#pragma unroll
          for (int u = 0; u < PB; ++u) {
            const int jj = jb + NKG * u;
            const float pj = jj < jn ? sp[jj] : 0.f;
            float x[VW];
            vec16<T>::cvt(vr[u], x);
#pragma unroll
            for (int e = 0; e < VW; ++e) oc[e] = fmaf(pj, x[e], oc[e]);
          }
          if (more) {
#pragma unroll
            for (int u = 0; u < PB; ++u) vr[u] = nx[u];
          }
        }
        __syncthreads();                       // sp and sred are reused
      }
#pragma unroll
      for (int e = 0; e < VW; ++e) so[kgp][ch * VW + e] = oc[e];
      __syncthreads();
      if (nsplit > 1) {
        // partial state of this split: max, sum, unnormalised P V row
        // (a split with no keys for this row leaves -inf, 0, 0)
        float* pr = part + (((size_t)b * Hq + h) * Tn + t) * nsplit * (D + 2) + (size_t)sp_id * (D + 2);
        if (tid < D) {
          float od = 0.f;
          for (int g = 0; g < NKG; ++g) od += so[g][tid];
          pr[2 + tid] = od;
        }
        if (tid == 0) { pr[0] = m; pr[1] = l; }
      } else if (tid < D) {
        float od = 0.f;
        for (int g = 0; g < NKG; ++g) od += so[g][tid];
        // retrieval from the state before this segment: sigma(q) M / (sigma(q) z + eps)
        float num = 0.f, den = 0.f;
        if (M) {
          const float* Mb = M + (size_t)bk * D * D;
          const float* zb = z + (size_t)bk * D;
#pragma unroll 16
          for (int a = 0; a < D; ++a) {
            const float sa = elu1(sq[a]);
            num = fmaf(sa, Mb[(size_t)a * D + tid], num);
            den = fmaf(sa, zb[a], den);
          }
        }
        den += 1e-6f;
        io<T>::store(O, qrow + tid, gt * (num / den) + (1.f - gt) * (od / l));
      }
      __syncthreads();                         // sq and so are reused
    }
  }
}

// Merge the key splits of one query row (max, sum and P V row of each),
// then retrieval from the state before the segment and the gate.  One
// workgroup of 256 threads per (batch, query head, new row): thread (g, c)
// owns output column c for split group g (splits g, g + NG, ...) and state
// rows g*RA .. g*RA+RA-1, so that every load the row needs is issued at once
// and waited for once; the groups' partial sums meet in LDS.
template <typename T, int D>
__global__ __launch_bounds__(DC_THREADS) void decode_combine_kernel(
    const T* __restrict__ Q, const float* __restrict__ beta, const float* __restrict__ M,
    const float* __restrict__ z, const float* __restrict__ part, T* __restrict__ O,
    int Hq, int Hkv, int Tn, int nsplit) {
  constexpr int NG = DC_THREADS / D;           // thread groups
  constexpr int RA = D / NG;                   // state rows per group
  constexpr int NS = (kDecodeMaxSplits + NG - 1) / NG;   // splits per group, at most
  __shared__ float rsum[4][NG][D];             // num, den, P V, sum
  __shared__ float rmax[NG];
  const int row = blockIdx.x;                  // (b * Hq + h) * Tn + t
  const int h = (row / Tn) % Hq, b = row / (Tn * Hq);
  const int bk = b * Hkv + h / (Hq / Hkv);
  const int c = threadIdx.x % D, g = threadIdx.x / D;
  const float* pr = part + (size_t)row * nsplit * (D + 2);
  // split parts: indexes past nsplit repeat the last split and get weight 0
  float pm[NS], pl[NS], po[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    const int s = min(g + NG * n, nsplit - 1);
    pm[n] = pr[s * (D + 2)];
    pl[n] = pr[s * (D + 2) + 1];
    po[n] = pr[s * (D + 2) + 2 + c];
  }
  float num = 0.f, den = 0.f;
  if (M) {
    const float* Mb = M + (size_t)bk * D * D;
    const float* zb = z + (size_t)bk * D;
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      const int a = g * RA + i;
      const float sa = elu1(io<T>::load(Q, (size_t)row * D + a));
      num = fmaf(sa, Mb[(size_t)a * D + c], num);
      den = fmaf(sa, zb[a], den);
    }
  }
  float gm = pm[0];
#pragma unroll
  for (int n = 1; n < NS; ++n) gm = fmaxf(gm, pm[n]);
  if (c == 0) rmax[g] = gm;
  __syncthreads();
  float mx = rmax[0];                          // finite: split 0 holds key 0 of every row
#pragma unroll
  for (int i = 1; i < NG; ++i) mx = fmaxf(mx, rmax[i]);
  float l = 0.f, od = 0.f;
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    // a split with no keys for this row holds (-inf, 0, 0): weight 0
    const float w = g + NG * n < nsplit ? __expf(pm[n] - mx) : 0.f;
    l = fmaf(w, pl[n], l);
    od = fmaf(w, po[n], od);
  }
  rsum[0][g][c] = num;
  rsum[1][g][c] = den;
  rsum[2][g][c] = od;
  rsum[3][g][c] = l;
  __syncthreads();
  if (g == 0) {
#pragma unroll
    for (int i = 1; i < NG; ++i) {
      num += rsum[0][i][c];
      den += rsum[1][i][c];
      od += rsum[2][i][c];
      l += rsum[3][i][c];
    }
    den += 1e-6f;
    const float gt = sigmoid(beta[h]);
    io<T>::store(O, (size_t)row * D + c, gt * (num / den) + (1.f - gt) * (od / l));
  }
}

// Key splits per row: 1 when the (batch, K/V head) pairs already fill the
// chip, else enough splits of at least 128 keys to reach about 256
// workgroups (at most kDecodeMaxSplits).
int decode_splits(const Geometry& g, int keys) {
  const int units = g.B * g.Hkv;
  if (units >= 256) return 1;
  int n = (256 + units - 1) / units;
  const int most = (keys + 127) / 128;
  if (n > most) n = most;
  if (n > kDecodeMaxSplits) n = kDecodeMaxSplits;
  return n < 1 ? 1 : n;
}

size_t decode_partial_bytes(const Geometry& g, int Tn) {
  return (size_t)g.B * g.Hq * Tn * kDecodeMaxSplits * (g.D + 2) * 4;
}

template <typename T, int D>
static hipError_t decode_t(const Geometry& g, int Tn, int pos, const void* Q, const void* K,
                           const void* V, const float* beta, void* Kc, void* Vc, const float* M,
                           const float* z, void* O, float* part, hipStream_t st) {
  const int nsplit = decode_splits(g, pos + Tn);
  const int split_keys = nsplit == 1 ? g.L : (pos + Tn + nsplit - 1) / nsplit;
  hipLaunchKernelGGL((decode_kernel<T, D>), dim3(g.B * g.Hkv * nsplit), dim3(DC_THREADS), 0, st,
                     static_cast<const T*>(Q), static_cast<const T*>(K), static_cast<const T*>(V), beta,
                     static_cast<T*>(Kc), static_cast<T*>(Vc), M, z, static_cast<T*>(O), part, g.Hq, g.Hkv,
                     Tn, g.L, pos, nsplit, split_keys, 1.f / sqrtf((float)D));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(g.B * g.Hq * Tn), dim3(DC_THREADS), 0, st,
                     static_cast<const T*>(Q), beta, M, z, part, static_cast<T*>(O), g.Hq, g.Hkv, Tn, nsplit);
  return hipGetLastError();
}

hipError_t launch_decode(const Geometry& g, int Tn, int pos, const void* Q, const void* K, const void* V,
                         const float* beta, void* Kc, void* Vc, const float* M, const float* z, void* O,
                         float* part, hipStream_t st) {
  if (g.dtype == 0) {
    if (g.D == 32) return decode_t<float, 32>(g, Tn, pos, Q, K, V, beta, Kc, Vc, M, z, O, part, st);
    if (g.D == 64) return decode_t<float, 64>(g, Tn, pos, Q, K, V, beta, Kc, Vc, M, z, O, part, st);
    if (g.D == 128) return decode_t<float, 128>(g, Tn, pos, Q, K, V, beta, Kc, Vc, M, z, O, part, st);
  } else {
    if (g.D == 32) return decode_t<bf16_t, 32>(g, Tn, pos, Q, K, V, beta, Kc, Vc, M, z, O, part, st);
    if (g.D == 64) return decode_t<bf16_t, 64>(g, Tn, pos, Q, K, V, beta, Kc, Vc, M, z, O, part, st);
    if (g.D == 128) return decode_t<bf16_t, 128>(g, Tn, pos, Q, K, V, beta, Kc, Vc, M, z, O, part, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace infini
