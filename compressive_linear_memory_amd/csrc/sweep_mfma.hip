// Memory phase of the bf16 forward on the matrix cores (gfx950).
//
// The memory path (page "Hugging Face Infini-Attention 재현 분석", section
// "Infini-Attention 메커니즘", steps Memory Update and State Transfer) is a
// prefix sum over segments of per-segment terms that depend only on K and V:
//   dM_s = sigma(K_s)^T V_s        dz_s = sum_rows sigma(K_s)
//   M_{s-1} = M0 + sum_{t<s} dM_t  (the state segment s retrieves from)
// so it runs in two launches:
//   delta_mfma_kernel  one workgroup per (batch, K/V head, segment, key
//                      split): the split's part of dM_s on
//                      v_mfma_f32_32x32x16_bf16 with sigma(K)^T and V^T staged
//                      key-contiguous in LDS; dz_s in fp32 from the unrounded
//                      sigma(K).  Grids with few segments split each segment's
//                      keys over several workgroups so that the whole chip
//                      takes part; the scan adds the parts in a fixed order.
//   scan_kernel        one workgroup per 64x64 tile of M per (batch, K/V head):
//                      walks the segments in order with the tile resident in
//                      registers, publishes each M_{s-1} as a transposed bf16
//                      copy (the operand layout the attention kernel reads;
//                      optionally also its rounding remainder, for the
//                      backward's retrieval gradient) and z_{s-1} in fp32, and
//                      writes the final state.
#include <hip/hip_runtime.h>

#include "common.h"
#include "infini.h"
#include "kernels.h"

namespace infini {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int D>
struct DeltaCfg {
  static constexpr int BK = 64;            // keys per staged chunk
  static constexpr int TSTR = BK + 8;      // row stride of the key-contiguous tiles
  static constexpr int WT = D / 2;         // wave tile edge (4 waves in 2 x 2)
  static constexpr int WB = WT / 32;       // 32x32 blocks per wave tile edge
  static constexpr int KPT = D / 32;       // keys per thread in staging
  static constexpr int TILE = D * TSTR;    // one transposed tile (elements)
  static constexpr int NKG = 256 / (D / 8);   // key groups
};

// GROUPED: segment sl of the launch is segment sl % spc of call sl / spc,
// whose K and V `tab` holds.
template <int D, bool GROUPED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void delta_mfma_kernel(const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                       float* __restrict__ dM, float* __restrict__ dz,
                       int N, int L, int s_begin, int nseg, int nsplit, int split_keys,
                       FwdCallTable tab, int spc, const int* __restrict__ lens, int Hkv) {
  using C = DeltaCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 smem[4 * C::TILE];   // 2 buffers x (K^T, V^T)
  static_assert(C::NKG * (D + 1) * 4 <= 4 * C::TILE * 2, "dz reduction must fit the tile buffers");
  float (*zred)[D + 1] = reinterpret_cast<float (*)[D + 1]>(smem);     // reused after the key loop

  const int part = blockIdx.x;               // unit * nsplit + split
  const int unit = part / nsplit;            // (b * Hkv + kvh) * nseg + sl
  const int k_begin = (part % nsplit) * split_keys;
  const int sl = unit % nseg;
  const size_t bk = unit / nseg;
  int s = s_begin + sl;
  if constexpr (GROUPED) {
    const int c = sl / spc;
    s = sl % spc;
    K = tab.K[c]; V = tab.V[c];
  }
  const size_t base = (bk * N + (size_t)s * L + k_begin) * D;
  // keys of this split (may be none); the last segment may be short, and in
  // a variable-length batch the segment may lie past its sequence's end
  const int Nb = seq_len_of(lens, (int)(bk / Hkv), N);
  L = max(0, min(min(L, Nb - s * L) - k_begin, split_keys));

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 31, hh = lane >> 5;
  const int wa = wave >> 1, wc = wave & 1;
  // Staging: consecutive lanes take consecutive key groups, so the transposed
  // LDS stores of a 16-lane group fall in one row, in distinct banks.
  const int kg = tid % C::NKG, dc = tid / C::NKG;

  float zp[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) zp[e] = 0.f;
  bf16x8_t kst[C::KPT], vst[C::KPT];

  auto load_chunk = [&](int j0) {
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int key = j0 + kg * C::KPT + i;
      bf16x8_t kv = {}, vv = {};
      if (key < L) {
        kv = *reinterpret_cast<const bf16x8_t*>(K + base + (size_t)key * D + dc * 8);
        vv = *reinterpret_cast<const bf16x8_t*>(V + base + (size_t)key * D + dc * 8);
      }
      kst[i] = kv;
      vst[i] = vv;
    }
  };
  auto store_chunk = [&](int buf, int j0) {
    __bf16* Kt = smem + buf * 2 * C::TILE;
    __bf16* Vt = Kt + C::TILE;
    float sk[C::KPT][8];
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const bool in = j0 + kg * C::KPT + i < L;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = in ? elu1((float)kst[i][e]) : 0.f;
        sk[i][e] = f;
        zp[e] += f;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16* kd = Kt + (dc * 8 + e) * C::TSTR + kg * C::KPT;
      __bf16* vd = Vt + (dc * 8 + e) * C::TSTR + kg * C::KPT;
      if constexpr (C::KPT == 4) {
        *reinterpret_cast<bf16x4_t*>(kd) = bf16x4_t{(__bf16)sk[0][e], (__bf16)sk[1][e], (__bf16)sk[2][e], (__bf16)sk[3][e]};
        *reinterpret_cast<bf16x4_t*>(vd) = bf16x4_t{vst[0][e], vst[1][e], vst[2][e], vst[3][e]};
      } else {
        *reinterpret_cast<bf16x2_t*>(kd) = bf16x2_t{(__bf16)sk[0][e], (__bf16)sk[1][e]};
        *reinterpret_cast<bf16x2_t*>(vd) = bf16x2_t{vst[0][e], vst[1][e]};
      }
    }
  };

  f32x16_t acc[C::WB][C::WB];
#pragma unroll
  for (int x = 0; x < C::WB; ++x)
#pragma unroll
    for (int y = 0; y < C::WB; ++y) acc[x][y] = f32x16_t{};

  const int nch = (L + C::BK - 1) / C::BK;
  if (nch > 0) {
    load_chunk(0);
    store_chunk(0, 0);
  }
  __syncthreads();
  for (int j = 0; j < nch; ++j) {
    if (j + 1 < nch) load_chunk((j + 1) * C::BK);
    const __bf16* Kt = smem + (j & 1) * 2 * C::TILE;
    const __bf16* Vt = Kt + C::TILE;
#pragma unroll
    for (int ks = 0; ks < C::BK / 16; ++ks) {
      bf16x8_t a[C::WB], bb[C::WB];
#pragma unroll
      for (int x = 0; x < C::WB; ++x) {
        a[x] = *reinterpret_cast<const bf16x8_t*>(Kt + (wa * C::WT + x * 32 + lq) * C::TSTR + ks * 16 + hh * 8);
        bb[x] = *reinterpret_cast<const bf16x8_t*>(Vt + (wc * C::WT + x * 32 + lq) * C::TSTR + ks * 16 + hh * 8);
      }
#pragma unroll
      for (int x = 0; x < C::WB; ++x)
#pragma unroll
        for (int y = 0; y < C::WB; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x], bb[y], acc[x][y], 0, 0, 0);
    }
    if (j + 1 < nch) store_chunk((j + 1) & 1, (j + 1) * C::BK);
    __syncthreads();
  }

  // dM[a][c]: lane holds column c = lq, rows 8(r/4) + 4hh + r%4 of each block.
  float* out = dM + (size_t)part * D * D;
#pragma unroll
  for (int x = 0; x < C::WB; ++x)
#pragma unroll
    for (int y = 0; y < C::WB; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int a = wa * C::WT + x * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        const int c = wc * C::WT + y * 32 + lq;
        out[(size_t)a * D + c] = acc[x][y][r];
      }
  // dz: reduce the per-thread partial sums over key groups.
#pragma unroll
  for (int e = 0; e < 8; ++e) zred[kg][dc * 8 + e] = zp[e];
  __syncthreads();
  for (int a = tid; a < D; a += 256) {
    float t = 0.f;
    for (int g = 0; g < C::NKG; ++g) t += zred[g][a];
    dz[(size_t)part * D + a] = t;
  }
}

// ---------------------------------------------------------------- scan

constexpr int SC_T = 32;   // tile edge: (D/32)^2 workgroups per (b, K/V head)
constexpr int SC_E = SC_T * SC_T / 256;   // state elements per thread
constexpr int SC_W = SC_T / SC_E;         // threads per tile row
static_assert(SC_E == 4, "one float4 of state and one bf16x4 of the transposed snapshot per thread");

template <int D>
__global__ __launch_bounds__(256) void scan_kernel(
    const float* __restrict__ dM, const float* __restrict__ dz, const float* M_in, const float* z_in,
    float* M_out, float* z_out, __bf16* __restrict__ MsnapT, float* __restrict__ zsnap, int nseg,
    int nsplit, __bf16* __restrict__ MsnapTlo) {
  constexpr int TPR = D / SC_T;
  __shared__ float tr[SC_T][SC_T + 1];
  const int a0 = (blockIdx.x / TPR) * SC_T, c0 = (blockIdx.x % TPR) * SC_T;
  const bool do_z = (blockIdx.x % TPR) == 0;
  const size_t bk = blockIdx.y;
  const int tid = threadIdx.x;
  const int ra = tid / SC_W, rc = (tid % SC_W) * SC_E;   // row a0+ra, columns c0+rc..+SC_E-1
  const size_t eoff = (size_t)(a0 + ra) * D + c0 + rc;

  float run[SC_E];
#pragma unroll
  for (int x = 0; x < SC_E; ++x) run[x] = M_in ? M_in[bk * D * D + eoff + x] : 0.f;
  float zr = 0.f;
  if (do_z && tid < SC_T) zr = z_in ? z_in[bk * D + a0 + tid] : 0.f;

  for (int sl = 0; sl < nseg; ++sl) {
    const size_t unit = bk * nseg + sl;
    // dM_s = sum of its key-split parts, added in split order.  The loads are
    // issued before M_{s-1} is published so that they overlap the transpose.
    float part[SC_E];
#pragma unroll 4
    for (int sp = 0; sp < nsplit; ++sp) {
      const float* src = dM + (unit * nsplit + sp) * D * D + eoff;
#pragma unroll
      for (int x = 0; x < SC_E; x += 4) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(src + x);
        if (sp == 0) {
          part[x] = v[0]; part[x + 1] = v[1]; part[x + 2] = v[2]; part[x + 3] = v[3];
        } else {
          part[x] += v[0]; part[x + 1] += v[1]; part[x + 2] += v[2]; part[x + 3] += v[3];
        }
      }
    }
    float zpart = 0.f;
    if (do_z && tid < SC_T) {
      zpart = dz[(unit * nsplit) * D + a0 + tid];
#pragma unroll 4
      for (int sp = 1; sp < nsplit; ++sp) zpart += dz[(unit * nsplit + sp) * D + a0 + tid];
    }
    // publish M_{s-1} transposed in bf16: stage the fp32 tile, read columns
#pragma unroll
    for (int x = 0; x < SC_E; ++x) tr[ra][rc + x] = run[x];
    if (do_z && tid < SC_T) zsnap[unit * D + a0 + tid] = zr;
    __syncthreads();
    {
      const int cc = tid / SC_W, aa = (tid % SC_W) * SC_E;   // output row c0+cc, columns a0+aa..
      __bf16* dst = MsnapT + unit * D * D + (size_t)(c0 + cc) * D + a0 + aa;
      bf16x4_t w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)tr[aa + e][cc];
      *reinterpret_cast<bf16x4_t*>(dst) = w;
      if (MsnapTlo) {   // the rounding remainder, for readers that need M beyond bf16
        bf16x4_t lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) lo[e] = (__bf16)(tr[aa + e][cc] - (float)w[e]);
        *reinterpret_cast<bf16x4_t*>(MsnapTlo + (dst - MsnapT)) = lo;
      }
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < SC_E; ++x) run[x] += part[x];
    if (do_z && tid < SC_T) zr += zpart;
  }
  if (M_out) {
#pragma unroll
    for (int x = 0; x < SC_E; ++x) M_out[bk * D * D + eoff + x] = run[x];
    if (do_z && tid < SC_T) z_out[bk * D + a0 + tid] = zr;
  }
}

template <int D>
static hipError_t sweep_mfma_t(const Geometry& g, const void* K, const void* V, const float* M_in,
                               const float* z_in, float* M_out, float* z_out, float* dM, float* dz,
                               void* MsnapT, float* zsnap, int s_begin, int s_end, hipStream_t st,
                               void* MsnapTlo) {
  const int nseg = s_end - s_begin;
  const int nsplit = delta_splits(g);
  const int split_keys = (((g.L + nsplit - 1) / nsplit + 63) / 64) * 64;
  const long long parts = (long long)g.B * g.Hkv * nseg * nsplit;
  if (parts > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((delta_mfma_kernel<D, false>), dim3((unsigned)parts), dim3(256), 0, st,
                     static_cast<const __bf16*>(K), static_cast<const __bf16*>(V), dM, dz, g.N, g.L,
                     s_begin, nseg, nsplit, split_keys, FwdCallTable{}, 1, g.lens, g.Hkv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid((D / SC_T) * (D / SC_T), g.B * g.Hkv);
  hipLaunchKernelGGL((scan_kernel<D>), grid, dim3(256), 0, st, dM, dz, M_in, z_in, M_out, z_out,
                     static_cast<__bf16*>(MsnapT), zsnap, nseg, nsplit, static_cast<__bf16*>(MsnapTlo));
  return hipGetLastError();
}

// Key splits per segment for the delta kernel: 1 when a chunk of segments
// already gives every compute unit work, else enough splits of at least 128
// keys to reach about 512 workgroups.
int delta_splits(const Geometry& g) {
  const long long units = (long long)g.B * g.Hkv * (g.S < INFINI_CHUNK_SEGMENTS ? g.S : INFINI_CHUNK_SEGMENTS);
  if (units == 0 || units >= 256) return 1;   // units = 0: an empty problem
  const long long want = (512 + units - 1) / units;
  const long long most = g.L / 128 > 1 ? g.L / 128 : 1;
  const long long n = want < most ? want : most;
  return (int)(n < 16 ? n : 16);
}

template <int D>
static hipError_t sweep_mfma_group_t(const Geometry& g, const FwdCallTable& tab, int ncalls, const float* M_in,
                                     const float* z_in, float* M_out, float* z_out, float* dM, float* dz,
                                     void* MsnapT, float* zsnap, hipStream_t st) {
  // the calls' segments as one run, each split as a single call's memory
  // phase splits it (same parts, same summation order)
  const int nseg = ncalls * g.S;
  const int nsplit = delta_splits(g);
  const int split_keys = (((g.L + nsplit - 1) / nsplit + 63) / 64) * 64;
  const long long parts = (long long)g.B * g.Hkv * nseg * nsplit;
  if (parts > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((delta_mfma_kernel<D, true>), dim3((unsigned)parts), dim3(256), 0, st, nullptr, nullptr, dM,
                     dz, g.N, g.L, 0, nseg, nsplit, split_keys, tab, g.S, nullptr, g.Hkv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid((D / SC_T) * (D / SC_T), g.B * g.Hkv);
  hipLaunchKernelGGL((scan_kernel<D>), grid, dim3(256), 0, st, dM, dz, M_in, z_in, M_out, z_out,
                     static_cast<__bf16*>(MsnapT), zsnap, nseg, nsplit, nullptr);
  return hipGetLastError();
}

hipError_t launch_sweep_mfma_group(const Geometry& g, const FwdCallTable& tab, int ncalls, const float* M_in,
                                   const float* z_in, float* M_out, float* z_out, float* dM, float* dz,
                                   void* MsnapT, float* zsnap, hipStream_t st) {
  if (g.dtype != 1 || ncalls < 1 || ncalls > kFwdMaxGroup) return hipErrorInvalidValue;
  if (g.D == 128) return sweep_mfma_group_t<128>(g, tab, ncalls, M_in, z_in, M_out, z_out, dM, dz, MsnapT, zsnap, st);
  if (g.D == 64) return sweep_mfma_group_t<64>(g, tab, ncalls, M_in, z_in, M_out, z_out, dM, dz, MsnapT, zsnap, st);
  return hipErrorInvalidValue;
}

hipError_t launch_sweep_mfma(const Geometry& g, const void* K, const void* V, const float* M_in,
                             const float* z_in, float* M_out, float* z_out, float* dM, float* dz,
                             void* MsnapT, float* zsnap, int s_begin, int s_end, hipStream_t st,
                             void* MsnapTlo) {
  if (g.dtype != 1) return hipErrorInvalidValue;
  if (g.D == 128) return sweep_mfma_t<128>(g, K, V, M_in, z_in, M_out, z_out, dM, dz, MsnapT, zsnap, s_begin, s_end, st, MsnapTlo);
  if (g.D == 64) return sweep_mfma_t<64>(g, K, V, M_in, z_in, M_out, z_out, dM, dz, MsnapT, zsnap, s_begin, s_end, st, MsnapTlo);
  return hipErrorInvalidValue;
}

}  // namespace infini
