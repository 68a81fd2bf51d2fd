// Backward of the bf16 Infini-attention segment kernel for segments longer
// than the fused short backward takes, on the matrix cores (gfx950).
//
// It is the same derivative as the generic backward (page "Hugging Face
// Infini-Attention 재현 분석", section "Infini-Attention 메커니즘": Local
// Attention, Memory Retrieval, Integration, Memory Update; the gradient
// formulas are listed at the top of generic_bwd.hip) and writes the same
// per-row workspace, so the pieces of either path can follow each other.
//
// bwd_q_mfma_kernel: one workgroup per (query tile, head, segment); each wave
// owns 32 query rows and every product is transposed so that a lane owns one
// query row (layouts as in fwd_mfma.hip):
//   pass 1   S^T = K Q^T, P from the row log-sum-exp (given, or formed by an
//            online softmax), A_dot^T = V^T P^T
//   retrieval  A_mem^T = M^T sigma(Q)^T with M_{s-1} as a bf16 hi/lo pair (the
//            retrieval gradient is a difference of nearly equal terms), den,
//            dnum = g dO / den, dden, D_i = rowsum(dA_dot * A_dot), the gate
//            term, and dQ^T = (M dnum^T + z dden^T) * sigma'(Q)^T
//   pass 2   dP^T = V dA_dot^T, dS = P (dP - D_i) / sqrt(d), dQ^T += K^T dS^T
// bwd_kv_mfma_kernel: one workgroup per (key tile, K/V head, segment); each
// wave owns 32 keys, a lane one key (the products transposed the other way):
//   per query head of the group and 64-row query tile at or after the keys:
//            S = Q K^T, P from the row log-sum-exp, dP = dA_dot V^T,
//            dS = P (dP - D_i) / sqrt(d), dV^T += dA_dot^T P, dK^T += Q^T dS
//   update   dV^T += dM^T sigma(K)^T, dK^T += (dM V^T + dz) * sigma'(K)^T with
//            dM = dL/dM_s (bf16) and dz = dL/dz_s
// rdelta_mfma_kernel / rscan_rev_kernel: the gradient with respect to the
// state after every segment (see below).
// The transposed operands (V^T in pass 1, M, K^T, dA_dot^T, Q^T and dM^T in
// the gradient products) come from row-major LDS tiles through
// ds_read_b64_tr_b16.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace infini {

typedef __bf16 lbf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 lbf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 lbf16x2 __attribute__((ext_vector_type(2)));
typedef short ls16x4 __attribute__((ext_vector_type(4)));
typedef float lf32x16 __attribute__((ext_vector_type(16)));
typedef float lf32x4 __attribute__((ext_vector_type(4)));

template <int D>
struct BqCfg {
  // 4 waves of 32 query rows, two workgroups per compute unit (two waves per
  // SIMD; one wave per SIMD with the whole register file was 1.25x slower)
  static constexpr int BM = 128;                    // query rows per workgroup
  static constexpr int WPE = 2;                     // waves per SIMD
  static constexpr int NW = BM / 32;                // waves
  static constexpr int NT = NW * 64;
  // keys per tile: at head_dim 128, 32 keep the staging registers down
  static constexpr int BN = D == 128 ? 32 : 64;
  static constexpr int NKB = BN / 32;               // 32-key blocks per tile
  static constexpr int KS = D / 16;                 // k-steps over head_dim
  static constexpr int DB = D / 32;                 // 32-row blocks of head_dim
  static constexpr int KSTR = D + 8;                // row stride of the K and V tiles
  static constexpr int KTILE = BN * KSTR;
  static constexpr int BUF = 2 * KTILE;             // K tile, V tile
  static constexpr int CPT = BN * D / 8 / NT;       // 16-byte chunks per thread per tile
  static constexpr int MSTR = D + 8;                // row stride of the M^T hi / lo tiles
  static constexpr int LDS = (2 * BUF > 2 * D * MSTR) ? 2 * BUF : 2 * D * MSTR;
};

__device__ __forceinline__ float lpair_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lpair_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// gfx950 transposing LDS read: in each group of 16 lanes, lane j receives
// element j % 4 of the four 4-element pieces addressed by lanes j/4, j/4 + 4,
// j/4 + 8 and j/4 + 12.
__device__ __forceinline__ lbf16x4 ltr4(const __bf16* p) {
  return __builtin_bit_cast(lbf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) ls16x4*)(p)));
}

// A operand (row r = r0 + lane % 16 of X^T, X row-major [k][r] with row stride
// xs) of a 32x32x16 product whose k-slots hold the keys k0 + e (e < 4) and
// k1 + e - 4 (e >= 4); r0 and k0 / k1 depend on the lane's group of 16.
__device__ __forceinline__ lbf16x8 ltr_op(const __bf16* X, int xs, int r0, int k0, int k1, int lane) {
  const int i = lane & 15;
  const int e = i >> 2, a = i & 3;
  const lbf16x4 lo = ltr4(X + (k0 + e) * xs + r0 + 4 * a);
  const lbf16x4 hi = ltr4(X + (k1 + e) * xs + r0 + 4 * a);
  return lbf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <int D>
__global__ __launch_bounds__(BqCfg<D>::NT) __attribute__((amdgpu_waves_per_eu(BqCfg<D>::WPE, BqCfg<D>::WPE)))
void bwd_q_mfma_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                       const __bf16* __restrict__ V, const float* __restrict__ beta,
                       const __bf16* __restrict__ MhiT, const __bf16* __restrict__ MloT,
                       const float* __restrict__ zsnap, const __bf16* __restrict__ dO, __bf16* __restrict__ dQ,
                       float* __restrict__ ws_lse, float* __restrict__ ws_Dd, float* __restrict__ ws_dden,
                       float* __restrict__ ws_dnum, float* __restrict__ dbeta_part,
                       const float* __restrict__ lse_in, int Hq, int Hkv, int N, int L, int s_begin,
                       int nseg, int nqt, float sl2, float scale, const int* __restrict__ lens) {
  using C = BqCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 smem[C::LDS];
  __shared__ float zs[D];
  __shared__ float wsum[C::NW];

  // a workgroup takes query tiles p and nqt - 1 - p, the shorter first, so
  // that every workgroup walks the same number of key tiles
  const int npair = (nqt + 1) / 2;
  const int per_qt = (int)gridDim.x / npair;         // (head, batch, segment) units per tile pair
  const int pr = (int)blockIdx.x / per_qt;
  const int rem = (int)blockIdx.x % per_qt;
  const int h = rem % Hq;
  const int sl = (rem / Hq) % nseg, b = (rem / Hq) / nseg;
  const int s = s_begin + sl;
  const int G = Hq / Hkv, kvh = h / G;
  int tid = threadIdx.x;
  // rows of this segment: the last may be short; none past the end of a
  // sequence of a variable-length batch (the gate partial is then zero)
  const int Ls = min(L, seq_len_of(lens, b, N) - s * L);
  for (int t = 0; t < 2; ++t) {
  // the lane-derived addresses are recomputed per tile instead of being held
  // (and spilled) across both
  asm volatile("" : "+v"(tid));
  const int qt = t == 0 ? pr : nqt - 1 - pr;
  if (t == 1) {
    if (qt == pr) break;          // the middle tile of an odd nqt goes alone
    __syncthreads();              // the first tile's LDS reads are done
  }
  const size_t dbp = (((size_t)b * Hq + h) * nseg + sl) * nqt + qt;
  if (Ls <= 0 || qt * C::BM >= Ls) {
    if (tid == 0) dbeta_part[dbp] = 0.f;
    continue;
  }
  const int lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 31, hh = lane >> 5;
  const int g16 = (lane >> 4) & 1;                // half of a 32-row block, for transposing reads
  const int q0 = qt * C::BM + wave * 32;
  const int qrow = q0 + lq;
  const bool qok = qrow < Ls;
  int qr = qok ? qrow : Ls - 1;
  const size_t qbase = (((size_t)b * Hq + h) * N + (size_t)s * L) * D;
  const size_t kvbase = (((size_t)b * Hkv + kvh) * N + (size_t)s * L) * D;
  const size_t crow = ((size_t)b * Hq + h) * ((size_t)nseg * L) + (size_t)sl * L + qrow;   // chunk row
  const float gt = sigmoid(beta[h]);

  // Q^T operand (lane: column qrow, k = 16 ks + 8 hh + e)
  lbf16x8 qreg[C::KS];
  {
    const __bf16* qp = Q + qbase + (size_t)qr * D + hh * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const lbf16x8 a = *reinterpret_cast<const lbf16x8*>(qp + ks * 16);
      qreg[ks] = qok ? a : lbf16x8{};
    }
  }

  const int kend = min(Ls, qt * C::BM + C::BM);
  const int ntiles = (kend + C::BN - 1) / C::BN;
  const bool live = q0 < Ls;

  // ---- staging of K and V tiles (row-major, both), double-buffered
  lbf16x8 kst[C::CPT], vst[C::CPT];
  constexpr int KRS = C::NT / (D / 8);
  const int krow0 = tid / (D / 8), kcol = (tid % (D / 8)) * 8;
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int key = min(k0 + krow0 + i * KRS, Ls - 1);
      kst[i] = *reinterpret_cast<const lbf16x8*>(K + kvbase + (size_t)key * D + kcol);
      vst[i] = *reinterpret_cast<const lbf16x8*>(V + kvbase + (size_t)key * D + kcol);
    }
  };
  auto store_tile = [&](int buf) {
    __bf16* Ks = smem + buf * C::BUF;
    __bf16* Vs = Ks + C::KTILE;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      *reinterpret_cast<lbf16x8*>(Ks + (krow0 + i * KRS) * C::KSTR + kcol) = kst[i];
      *reinterpret_cast<lbf16x8*>(Vs + (krow0 + i * KRS) * C::KSTR + kcol) = vst[i];
    }
  };
  // scores of one tile (S^T, C layout: column qrow, element (kb, r) is key
  // k0 + kb*32 + 8(r/4) + 4hh + r%4), masked past the diagonal and the segment end
  auto scores = [&](const __bf16* Ks, int k0, lf32x16 (&sacc)[C::NKB]) {
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      sacc[kb] = lf32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const lbf16x8 a = *reinterpret_cast<const lbf16x8*>(Ks + (kb * 32 + lq) * C::KSTR + ks * 16 + hh * 8);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], sacc[kb], 0, 0, 0);
      }
    }
    if (k0 + C::BN - 1 > q0 || k0 + C::BN > Ls) {
      const int lim = min(qrow, Ls - 1) - (k0 + 4 * hh);
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) sacc[kb][r] = -INFINITY;
    }
  };
  // one sweep over the key tiles, `step` called on each tile the wave attends to
  auto sweep = [&](auto&& step) {
    load_tile(0);
    store_tile(0);
    __syncthreads();
    if (ntiles > 1) load_tile(C::BN);
    for (int j = 0; j < ntiles; ++j) {
      const int k0 = j * C::BN;
      const __bf16* Ks = smem + (j & 1) * C::BUF;
      if (live && k0 <= q0 + 31) step(Ks, Ks + C::KTILE, k0);
      if (j + 1 < ntiles) store_tile((j + 1) & 1);
      __syncthreads();
      if (j + 2 < ntiles) load_tile((j + 2) * C::BN);
    }
  };

  // ---- pass 1: A_dot (and the row log-sum-exp unless given), base 2
  lf32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = lf32x16{};
  const bool have_lse = lse_in != nullptr;
  float m = have_lse ? lse_in[((size_t)b * Hq + h) * N + (size_t)s * L + qr] * 1.4426950408889634f : -INFINITY;
  float lpart = 0.f;
  const lbf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  sweep([&](const __bf16* Ks, const __bf16* Vs, int k0) {
    lf32x16 sacc[C::NKB];
    scores(Ks, k0, sacc);
    if (!have_lse) {
      float mt = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
      const float mn = fmaxf(m, lpair_max32(mt) * sl2);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      lpart *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
    }
    lbf16x8 pb[C::NKB][2];
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        pb[kb][r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[kb][r], sl2, -m));
    if (!have_lse) {
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int x = 0; x < 4; ++x)
            lpart = __builtin_amdgcn_fdot2_f32_bf16(lbf16x2{pb[kb][t][2 * x], pb[kb][t][2 * x + 1]}, ones, lpart, false);
    }
    // O^T += V^T P^T: k-slot x of half hh <-> key kb*32 + 16t + 8(x/4) + 4hh + x%4
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int kk = kb * 32 + 16 * t + 4 * hh;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const lbf16x8 a = ltr_op(Vs, C::KSTR, db * 32 + 16 * g16, kk, kk + 8, lane);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][t], oacc[db], 0, 0, 0);
        }
      }
  });
  float inv_l = 1.f;
  if (!have_lse) {
    const float l = lpair_sum32(lpart);
    inv_l = 1.f / l;
    m += __log2f(l);                          // m is now the row's log-sum-exp (base 2)
  }

  // ---- the terms that need A_dot: the gate partial's -dO.A_dot part and
  // D_i = rowsum(dA_dot * A_dot); A_dot is not held past them.  Per element
  // (cb, r) of the C layout: column c = cb*32 + 8(r/4) + 4hh + r%4
  float bsum = 0.f;
  float Dd;
  {
    float ddot = 0.f;
#pragma unroll
    for (int cb = 0; cb < C::DB; ++cb)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const lbf16x4 dv = *reinterpret_cast<const lbf16x4*>(dO + qbase + (size_t)qr * D + cb * 32 + 8 * u + 4 * hh);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          // rows past the segment end (a wave may have no key at all, l = 0)
          // contribute nothing
          const float go = qok ? (float)dv[x] : 0.f;
          const float ad = qok ? oacc[cb][4 * u + x] * inv_l : 0.f;
          // the row sum pairs with the rounded operand the dP products use,
          // so that dP - D_i cancels as it does exactly
          const __bf16 da = (__bf16)((1.f - gt) * go);
          bsum -= go * ad;
          ddot += (float)da * ad;
        }
      }
    Dd = lpair_sum32(ddot);
  }
  // (formed here: otherwise the compiler sinks the sum to its next use after
  // pass 2 and holds, and spills, the 128 terms it needs through the sweep)
  asm volatile("" : "+v"(bsum));
  // dA_dot^T operand = (1 - g) dO, rounded once (lane: column qrow)
  lbf16x8 dreg[C::KS];
  {
    const __bf16* dp = dO + qbase + (size_t)qr * D + hh * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const lbf16x8 d = *reinterpret_cast<const lbf16x8*>(dp + ks * 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) dreg[ks][e] = qok ? (__bf16)((1.f - gt) * (float)d[e]) : (__bf16)0.f;
    }
  }

  // ---- pass 2: dQ^T = K^T dS^T, dS = P (dP - D_i) / sqrt(d) with dP^T = V dA_dot^T
  // (rows a = ab*32 + 8(r/4) + 4hh + r%4)
  lf32x16 dq[C::DB];
#pragma unroll
  for (int ab = 0; ab < C::DB; ++ab) dq[ab] = lf32x16{};
  sweep([&](const __bf16* Ks, const __bf16* Vs, int k0) {
    lf32x16 sacc[C::NKB];
    scores(Ks, k0, sacc);
    lf32x16 pacc[C::NKB];
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      pacc[kb] = lf32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const lbf16x8 a = *reinterpret_cast<const lbf16x8*>(Vs + (kb * 32 + lq) * C::KSTR + ks * 16 + hh * 8);
        pacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dreg[ks], pacc[kb], 0, 0, 0);
      }
    }
    lbf16x8 dsb[C::NKB][2];
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], sl2, -m));
        dsb[kb][r >> 3][r & 7] = (__bf16)(scale * p * (pacc[kb][r] - Dd));
      }
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int kk = kb * 32 + 16 * t + 4 * hh;
#pragma unroll
        for (int ab = 0; ab < C::DB; ++ab) {
          const lbf16x8 a = ltr_op(Ks, C::KSTR, ab * 32 + 16 * g16, kk, kk + 8, lane);
          dq[ab] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb[kb][t], dq[ab], 0, 0, 0);
        }
      }
  });

  // (the retrieval reads dO again: passing the row index through an empty asm
  // keeps the compiler from holding the 64 unpacked values since the A_dot
  // terms in registers, and spilling them, instead)
  asm volatile("" : "+v"(qr));
  // ---- retrieval: M_{s-1}^T as bf16 hi / lo tiles [c][a] (published so by the
  // memory phase), z_{s-1}; the sweep's last barrier freed the tile buffers
  __bf16* Mhi = smem;
  __bf16* Mlo = smem + D * C::MSTR;
  {
    const size_t snap = ((size_t)(b * Hkv + kvh) * nseg + sl);
    for (int e = tid; e < D * D / 8; e += C::NT) {
      const int c = e / (D / 8), a = (e % (D / 8)) * 8;
      *reinterpret_cast<lbf16x8*>(Mhi + c * C::MSTR + a) = *reinterpret_cast<const lbf16x8*>(MhiT + snap * D * D + c * D + a);
      *reinterpret_cast<lbf16x8*>(Mlo + c * C::MSTR + a) = *reinterpret_cast<const lbf16x8*>(MloT + snap * D * D + c * D + a);
    }
    for (int e = tid; e < D; e += C::NT) zs[e] = zsnap[snap * D + e];
  }
  __syncthreads();
  lbf16x8 sq[C::KS];
  float dpart = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const __bf16 v = (__bf16)elu1((float)qreg[ks][e]);
      sq[ks][e] = v;
      dpart += (float)v * zs[ks * 16 + hh * 8 + e];
    }
  }
  const float den = lpair_sum32(dpart) + 1e-6f;
  const float inv_den = 1.f / den;
  float dmem = 0.f;
  lbf16x8 dnb[C::DB][2];                      // dnum^T operand, slots like the probabilities
#pragma unroll
  for (int cb = 0; cb < C::DB; ++cb) {
    lf32x16 nacc = {};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const lbf16x8 a = *reinterpret_cast<const lbf16x8*>(Mhi + (cb * 32 + lq) * C::MSTR + ks * 16 + hh * 8);
      const lbf16x8 al = *reinterpret_cast<const lbf16x8*>(Mlo + (cb * 32 + lq) * C::MSTR + ks * 16 + hh * 8);
      nacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sq[ks], nacc, 0, 0, 0);
      nacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, sq[ks], nacc, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c0 = cb * 32 + 8 * u + 4 * hh;
      const lbf16x4 dv = *reinterpret_cast<const lbf16x4*>(dO + qbase + (size_t)qr * D + c0);
      lf32x4 dn32;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = 4 * u + x;
        const float go = qok ? (float)dv[x] : 0.f;
        const float am = qok ? nacc[r] * inv_den : 0.f;
        // the row sum pairs with the rounded operand the products use, so that
        // dnum M^T + dden z^T cancel as they do exactly
        const __bf16 dn = (__bf16)(gt * go * inv_den);
        bsum += go * am;
        dmem += (float)dn * am;
        dnb[cb][r >> 3][r & 7] = dn;
        dn32[x] = gt * go * inv_den;
      }
      if (qok) *reinterpret_cast<lf32x4*>(ws_dnum + crow * D + c0) = dn32;
    }
    asm volatile("" : "+v"(bsum), "+v"(dmem));   // summed per block, not sunk to the end
    __builtin_amdgcn_sched_barrier(0);
  }
  const float dden = -lpair_sum32(dmem);
  if (qok && hh == 0) {
    ws_lse[crow] = m * 0.69314718055994531f;
    ws_Dd[crow] = Dd;
    ws_dden[crow] = dden;
  }
  // gate partial of the workgroup (fixed order)
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) bsum += __shfl_xor(bsum, o);
  if (lane == 0) wsum[wave] = bsum;

  // dQ^T += (M dnum^T + z dden) * sigma'(Q), M from M^T by transposing reads
#pragma unroll
  for (int ab = 0; ab < C::DB; ++ab) {
    lf32x16 ret = {};
#pragma unroll
    for (int cb = 0; cb < C::DB; ++cb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int kk = cb * 32 + 16 * t + 4 * hh;
        const lbf16x8 a = ltr_op(Mhi, C::MSTR, ab * 32 + 16 * g16, kk, kk + 8, lane);
        const lbf16x8 al = ltr_op(Mlo, C::MSTR, ab * 32 + 16 * g16, kk, kk + 8, lane);
        ret = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dnb[cb][t], ret, 0, 0, 0);
        ret = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, dnb[cb][t], ret, 0, 0, 0);
      }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int a0 = ab * 32 + 8 * u + 4 * hh;
      const lbf16x4 qv = *reinterpret_cast<const lbf16x4*>(Q + qbase + (size_t)qr * D + a0);
#pragma unroll
      for (int x = 0; x < 4; ++x)
        dq[ab][4 * u + x] += (ret[4 * u + x] + dden * zs[a0 + x]) * elu1_grad((float)qv[x]);
    }
  }
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int w = 0; w < C::NW; ++w) t += wsum[w];
    dbeta_part[dbp] = t;
  }

  if (qok) {
    __bf16* qp = dQ + qbase + (size_t)qrow * D;
#pragma unroll
    for (int ab = 0; ab < C::DB; ++ab)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        *reinterpret_cast<lbf16x4*>(qp + ab * 32 + 8 * u + 4 * hh) =
            lbf16x4{(__bf16)dq[ab][4 * u], (__bf16)dq[ab][4 * u + 1], (__bf16)dq[ab][4 * u + 2], (__bf16)dq[ab][4 * u + 3]};
  }
  }   // query tiles of the pair
}


template <int D>
struct BkCfg {
  static constexpr int BK = 128;                    // keys per workgroup (4 waves of 32)
  static constexpr int NT = 256;
  static constexpr int WPE = 2;                     // waves per SIMD
  // query rows per staged tile: at head_dim 128, 32 keep the staging registers
  // (and with them the spills) down
  static constexpr int BQ = D == 128 ? 32 : 64;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int QSTR = D + 8;                // row stride of the Q and dA_dot tiles
  static constexpr int QTILE = BQ * QSTR;
  static constexpr int BUF = 2 * QTILE;             // Q tile, dA_dot tile
  static constexpr int CPT = BQ * D / 8 / NT;       // 16-byte chunks per thread per tile
  static constexpr int MSTR = D + 8;                // row stride of the dM tile
  static constexpr int LDS = (2 * BUF > D * MSTR) ? 2 * BUF : D * MSTR;
  // at head_dim 128 the V^T operand is kept in LDS (lane-private, 16 bytes per
  // k-step and lane) rather than in registers, which the K^T operand and the
  // dK / dV accumulators fill
  static constexpr bool VSTASH = D == 128;
  static constexpr int VST = VSTASH ? NT * KS * 8 : 8;
};

template <int D>
__global__ __launch_bounds__(BkCfg<D>::NT) __attribute__((amdgpu_waves_per_eu(BkCfg<D>::WPE, BkCfg<D>::WPE)))
void bwd_kv_mfma_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                        const __bf16* __restrict__ V, const float* __restrict__ beta,
                        const __bf16* __restrict__ dO, const float* __restrict__ ws_lse,
                        const float* __restrict__ ws_Dd, const float* __restrict__ dMsnap,
                        const float* __restrict__ dzsnap, __bf16* __restrict__ dK, __bf16* __restrict__ dV,
                        int Hq, int Hkv, int N, int L, int s_begin, int nseg, float sl2, float scale,
                        const int* __restrict__ lens) {
  using C = BkCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 smem[C::LDS];
  __shared__ __attribute__((aligned(16))) float rowst[2][2][C::BQ];   // per buffer: lse (base 2), D_i
  __shared__ float dzs[D];
  __shared__ __attribute__((aligned(16))) __bf16 vstash[C::VST];

  // key tiles with the most query rows (the first) first
  const int per_kt = (int)gridDim.x / ((L + C::BK - 1) / C::BK);   // units per key tile
  const int kt = (int)blockIdx.x / per_kt;
  const int rem = (int)blockIdx.x % per_kt;
  const int kvh = rem % Hkv;
  const int sl = (rem / Hkv) % nseg, b = (rem / Hkv) / nseg;
  const int s = s_begin + sl;
  const int G = Hq / Hkv;
  // keys (and rows) of this segment: the last may be short; none past the end
  // of a sequence of a variable-length batch
  const int Ls = min(L, seq_len_of(lens, b, N) - s * L);
  const int k0 = kt * C::BK;
  if (Ls <= 0 || k0 >= Ls) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 31, hh = lane >> 5;
  const int g16 = (lane >> 4) & 1;
  const int kw = k0 + wave * 32;                    // this wave's first key
  const int key = kw + lq;                          // this lane's key (column of the products)
  const bool kok = key < Ls;
  const int kr = kok ? key : Ls - 1;
  const size_t kvbase = (((size_t)b * Hkv + kvh) * N + (size_t)s * L) * D;

  // K^T and V^T operands (lane: column key, k = 16 ks + 8 hh + e)
  lbf16x8 kreg[C::KS], vreg[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    kreg[ks] = *reinterpret_cast<const lbf16x8*>(K + kvbase + (size_t)kr * D + ks * 16 + hh * 8);
    vreg[ks] = *reinterpret_cast<const lbf16x8*>(V + kvbase + (size_t)kr * D + ks * 16 + hh * 8);
    if constexpr (C::VSTASH) *reinterpret_cast<lbf16x8*>(vstash + (ks * C::NT + tid) * 8) = vreg[ks];
  }
  // V^T operand k-step ks (lane-private: the lane reads back what it wrote)
  auto vop = [&](int ks) -> lbf16x8 {
    if constexpr (C::VSTASH) return *reinterpret_cast<const lbf16x8*>(vstash + (ks * C::NT + tid) * 8);
    else return vreg[ks];
  };
  lf32x16 dka[C::DB], dva[C::DB];                   // dK^T, dV^T: rows a = ab*32 + 8(r/4) + 4hh + r%4
#pragma unroll
  for (int db = 0; db < C::DB; ++db) { dka[db] = lf32x16{}; dva[db] = lf32x16{}; }

  // the (head, 64-row query tile) sequence: tiles from the one holding key k0
  const int qfirst = k0 / C::BQ;
  const int nqt = (Ls + C::BQ - 1) / C::BQ - qfirst;
  const int ntot = G * nqt;
  lbf16x8 qst[C::CPT], dst[C::CPT];
  float rl = 0.f, rd = 0.f;                         // this thread's lse / D_i staging (tid < BQ)
  constexpr int QRS = C::NT / (D / 8);
  const int qrow0 = tid / (D / 8), qcol = (tid % (D / 8)) * 8;
  auto tile_of = [&](int i, int& h, int& q0) {
    h = kvh * G + i / nqt;
    q0 = (qfirst + i % nqt) * C::BQ;
  };
  auto load_tile = [&](int i) {
    int h, q0;
    tile_of(i, h, q0);
    const size_t qbase = (((size_t)b * Hq + h) * N + (size_t)s * L) * D;
    const float og = 1.f - sigmoid(beta[h]);
#pragma unroll
    for (int x = 0; x < C::CPT; ++x) {
      const int row = min(q0 + qrow0 + x * QRS, Ls - 1);
      qst[x] = *reinterpret_cast<const lbf16x8*>(Q + qbase + (size_t)row * D + qcol);
      const lbf16x8 d = *reinterpret_cast<const lbf16x8*>(dO + qbase + (size_t)row * D + qcol);
      // dA_dot = (1 - g) dO, rounded once as the query side rounds it
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[x][e] = (__bf16)(og * (float)d[e]);
    }
    if (tid < C::BQ) {
      const int row = min(q0 + tid, Ls - 1);
      const size_t crow = ((size_t)b * Hq + h) * ((size_t)nseg * L) + (size_t)sl * L + row;
      rl = ws_lse[crow] * 1.4426950408889634f;
      rd = ws_Dd[crow];
    }
  };
  auto store_tile = [&](int buf) {
    __bf16* Qs = smem + buf * C::BUF;
    __bf16* As = Qs + C::QTILE;
#pragma unroll
    for (int x = 0; x < C::CPT; ++x) {
      *reinterpret_cast<lbf16x8*>(Qs + (qrow0 + x * QRS) * C::QSTR + qcol) = qst[x];
      *reinterpret_cast<lbf16x8*>(As + (qrow0 + x * QRS) * C::QSTR + qcol) = dst[x];
    }
    if (tid < C::BQ) {
      rowst[buf][0][tid] = rl;
      rowst[buf][1][tid] = rd;
    }
  };

  if (ntot > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  if (ntot > 1) load_tile(1);
  for (int i = 0; i < ntot; ++i) {
    const int buf = i & 1;
    int h, q0;
    tile_of(i, h, q0);
    const __bf16* Qs = smem + buf * C::BUF;
    const __bf16* As = Qs + C::QTILE;
#pragma unroll
    for (int qb = 0; qb < C::BQ / 32; ++qb) {
      const int qb0 = q0 + qb * 32;                 // first row of this 32-row block
      if (qb0 + 31 < kw || qb0 >= Ls) continue;     // every row before the wave's keys, or past the end
      // S[q][key] and dP[q][key]: element r holds row qb0 + 8(r/4) + 4hh + r%4
      lf32x16 sacc = {}, pacc = {};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const lbf16x8 qa = *reinterpret_cast<const lbf16x8*>(Qs + (qb * 32 + lq) * C::QSTR + ks * 16 + hh * 8);
        const lbf16x8 da = *reinterpret_cast<const lbf16x8*>(As + (qb * 32 + lq) * C::QSTR + ks * 16 + hh * 8);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kreg[ks], sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vop(ks), pacc, 0, 0, 0);
      }
      lbf16x8 pb[2], dsb[2];                        // k-slot x of half hh <-> row 16t + 8(x/4) + 4hh + x%4
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int rl0 = qb * 32 + 8 * u + 4 * hh;  // rows of elements 4u .. 4u+3
        const lf32x4 lse4 = *reinterpret_cast<const lf32x4*>(&rowst[buf][0][rl0]);
        const lf32x4 dd4 = *reinterpret_cast<const lf32x4*>(&rowst[buf][1][rl0]);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = 4 * u + x;
          const int row = q0 + rl0 + x;
          const bool on = row >= key && row < Ls;
          const float p = on ? __builtin_amdgcn_exp2f(fmaf(sacc[r], sl2, -lse4[x])) : 0.f;
          pb[r >> 3][r & 7] = (__bf16)p;
          dsb[r >> 3][r & 7] = (__bf16)(scale * p * (pacc[r] - dd4[x]));
        }
      }
      // dV^T += dA_dot^T P, dK^T += Q^T dS (contraction over the block's rows)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int rr = qb * 32 + 16 * t + 4 * hh;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const lbf16x8 aa = ltr_op(As, C::QSTR, db * 32 + 16 * g16, rr, rr + 8, lane);
          const lbf16x8 qa = ltr_op(Qs, C::QSTR, db * 32 + 16 * g16, rr, rr + 8, lane);
          dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aa, pb[t], dva[db], 0, 0, 0);
          dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, dsb[t], dka[db], 0, 0, 0);
        }
      }
    }
    if (i + 1 < ntot) store_tile((i + 1) & 1);
    __syncthreads();
    if (i + 2 < ntot) load_tile(i + 2);
  }

  // ---- update backward with dM = dL/dM_s: tile [a][c] (bf16), dz
  __bf16* dMs = smem;
  {
    const size_t snap = ((size_t)(b * Hkv + kvh) * nseg + sl);
    const float* src = dMsnap + snap * D * D;
    for (int e = tid; e < D * D; e += C::NT) dMs[(e / D) * C::MSTR + (e % D)] = (__bf16)src[e];
    for (int e = tid; e < D; e += C::NT) dzs[e] = dzsnap[snap * D + e];
  }
  __syncthreads();
  lbf16x8 sk[C::KS];                                // sigma(K)^T operand
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) sk[ks][e] = (__bf16)elu1((float)kreg[ks][e]);
  // dV^T[c][key] += sum_a dM[a][c] sigma(K)[key][a]: A = dM^T rows c through
  //   transposing reads of the [a][c] tile, k = a = 16 ks + 8 hh + e
  // (dM V^T)^T[a][key] = sum_c dM[a][c] V[key][c]: A = dM rows a (plain reads)
  lf32x16 dku[C::DB];
#pragma unroll
  for (int cb = 0; cb < C::DB; ++cb) {
    dku[cb] = lf32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const lbf16x8 a = ltr_op(dMs, C::MSTR, cb * 32 + 16 * g16, ks * 16 + 8 * hh, ks * 16 + 8 * hh + 4, lane);
      dva[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sk[ks], dva[cb], 0, 0, 0);
      const lbf16x8 am = *reinterpret_cast<const lbf16x8*>(dMs + (cb * 32 + lq) * C::MSTR + ks * 16 + hh * 8);
      dku[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, vop(ks), dku[cb], 0, 0, 0);
    }
  }
  // dK = Q^T dS (scaled) + (dM V^T + dz) sigma'(K); rows a of the accumulators
  // are ab*32 + 8(r/4) + 4hh + r%4
  if (kok) {
    __bf16* kp = dK + kvbase + (size_t)key * D;
    __bf16* vp = dV + kvbase + (size_t)key * D;
#pragma unroll
    for (int ab = 0; ab < C::DB; ++ab)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int a0 = ab * 32 + 8 * u + 4 * hh;
        const lbf16x4 kv = *reinterpret_cast<const lbf16x4*>(K + kvbase + (size_t)key * D + a0);
        lbf16x4 wk, wv;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = 4 * u + x;
          wk[x] = (__bf16)(dka[ab][r] + (dku[ab][r] + dzs[a0 + x]) * elu1_grad((float)kv[x]));
          wv[x] = (__bf16)dva[ab][r];
        }
        *reinterpret_cast<lbf16x4*>(kp + a0) = wk;
        *reinterpret_cast<lbf16x4*>(vp + a0) = wv;
      }
  }
}


// ---- reverse state scan on the matrix cores
//
// dL/dM_s (the state after segment s) is the upstream gradient plus the
// retrieval terms of every later segment, R_t = sum over the group's heads and
// the segment's rows of sigma(Q)^T dnum (and r_t = sigma(Q)^T dden for z):
//   rdelta_mfma_kernel  one workgroup per (batch, K/V head, segment): R_s, r_s
//   rscan_rev_kernel    one workgroup per 32x32 tile of the state per (batch,
//                       K/V head): walks the segments last to first, publishing
//                       dL/dM_s before adding R_s, and writes the gradient
//                       with respect to the state the chunk started from.
template <int D>
struct RdCfg {
  static constexpr int BR = 64;                     // rows per staged tile
  static constexpr int STR = D + 8;
  static constexpr int CPT = BR * D / 8 / 256;      // 8-element chunks per thread per tile
  static constexpr int WB = D / 64;                 // 32-blocks per wave edge (2x2 waves)
};

template <int D>
__global__ __launch_bounds__(256) void rdelta_mfma_kernel(
    const __bf16* __restrict__ Q, const float* __restrict__ dnum, const float* __restrict__ dden,
    float* __restrict__ R, float* __restrict__ r, int Hq, int Hkv, int N, int L, int s_begin, int nseg,
    const int* __restrict__ lens) {
  using C = RdCfg<D>;
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  __shared__ __attribute__((aligned(16))) __bf16 SQ[C::BR * C::STR];   // sigma(Q) rows
  __shared__ __attribute__((aligned(16))) __bf16 DN[C::BR * C::STR];   // dnum rows
  __shared__ float dd[C::BR];
  const int unit = blockIdx.x;                      // bk * nseg + sl
  const int sl = unit % nseg;
  const int bk = unit / nseg;
  const int b = bk / Hkv, kvh = bk % Hkv;
  const int G = Hq / Hkv;
  const int s = s_begin + sl;
  const int Ls = max(0, min(L, seq_len_of(lens, b, N) - s * L));
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 31, hh = lane >> 5;
  const int g16 = (lane >> 4) & 1;
  // this wave's blocks of R: rows a = (2 (wave >> 1) + ..)..., columns c likewise
  const int a_base = (wave >> 1) * (D / 2), c_base = (wave & 1) * (D / 2);
  lf32x16 acc[C::WB][C::WB];
#pragma unroll
  for (int x = 0; x < C::WB; ++x)
#pragma unroll
    for (int y = 0; y < C::WB; ++y) acc[x][y] = lf32x16{};
  float zacc = 0.f;                                  // r[a] for a = tid (< D)
  constexpr int RS8 = 256 / (D / 8);
  const int row0 = tid / (D / 8), col = (tid % (D / 8)) * 8;
  for (int h = kvh * G; h < (kvh + 1) * G; ++h) {
    const size_t qbase = (((size_t)b * Hq + h) * N + (size_t)s * L) * D;
    const size_t cbase = ((size_t)b * Hq + h) * ((size_t)nseg * L) + (size_t)sl * L;
    for (int i0 = 0; i0 < Ls; i0 += C::BR) {
#pragma unroll
      for (int x = 0; x < C::CPT; ++x) {
        const int row = row0 + x * RS8;
        const bool in = i0 + row < Ls;
        lbf16x8 sq = {}, dn = {};
        if (in) {
          const lbf16x8 qv = *reinterpret_cast<const lbf16x8*>(Q + qbase + (size_t)(i0 + row) * D + col);
          const lf32x4 d0 = *reinterpret_cast<const lf32x4*>(dnum + (cbase + i0 + row) * D + col);
          const lf32x4 d1 = *reinterpret_cast<const lf32x4*>(dnum + (cbase + i0 + row) * D + col + 4);
#pragma unroll
          for (int e = 0; e < 8; ++e) sq[e] = (__bf16)elu1((float)qv[e]);
#pragma unroll
          for (int e = 0; e < 4; ++e) { dn[e] = (__bf16)d0[e]; dn[e + 4] = (__bf16)d1[e]; }
        }
        *reinterpret_cast<lbf16x8*>(SQ + row * C::STR + col) = sq;
        *reinterpret_cast<lbf16x8*>(DN + row * C::STR + col) = dn;
      }
      if (tid < C::BR) dd[tid] = (i0 + tid < Ls) ? dden[cbase + i0 + tid] : 0.f;
      __syncthreads();
      // R[a][c] += sum_q sigma(Q)[q][a] dnum[q][c]; both operands by transposing
      // reads, k-slot e of half hh <-> row 16 kk + 8 hh + e
#pragma unroll
      for (int kk = 0; kk < C::BR / 16; ++kk) {
        lbf16x8 bo[C::WB];
#pragma unroll
        for (int y = 0; y < C::WB; ++y)
          bo[y] = ltr_op(DN, C::STR, c_base + y * 32 + 16 * g16, kk * 16 + 8 * hh, kk * 16 + 8 * hh + 4, lane);
#pragma unroll
        for (int x = 0; x < C::WB; ++x) {
          const lbf16x8 ao = ltr_op(SQ, C::STR, a_base + x * 32 + 16 * g16, kk * 16 + 8 * hh, kk * 16 + 8 * hh + 4, lane);
#pragma unroll
          for (int y = 0; y < C::WB; ++y)
            acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, bo[y], acc[x][y], 0, 0, 0);
        }
      }
      if (tid < D) {
        float t4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int q = 0; q < C::BR; ++q) t4[q & 3] += (float)SQ[q * C::STR + tid] * dd[q];
        zacc += (t4[0] + t4[1]) + (t4[2] + t4[3]);
      }
      __syncthreads();
    }
  }
  // C layout: column c = c_base + y*32 + lq, rows a = a_base + x*32 + 8(e/4) + 4hh + e%4
  float* Rs = R + (size_t)unit * D * D;
#pragma unroll
  for (int x = 0; x < C::WB; ++x)
#pragma unroll
    for (int y = 0; y < C::WB; ++y)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        Rs[(size_t)(a_base + x * 32 + 8 * (e >> 2) + 4 * hh + (e & 3)) * D + c_base + y * 32 + lq] = acc[x][y][e];
  if (tid < D) r[(size_t)unit * D + tid] = zacc;
}

template <int D>
__global__ __launch_bounds__(256) void rscan_rev_kernel(
    const float* __restrict__ R, const float* __restrict__ r, const float* dM_in, const float* dz_in,
    float* dM_out, float* dz_out, float* __restrict__ dMsnap, float* __restrict__ dzsnap, int nseg) {
  constexpr int T = 32, TPR = D / T;
  const int a0 = (blockIdx.x / TPR) * T, c0 = (blockIdx.x % TPR) * T;
  const bool do_z = (blockIdx.x % TPR) == 0;
  const size_t bk = blockIdx.y;
  const int tid = threadIdx.x;
  const size_t eoff = (size_t)(a0 + tid / 8) * D + c0 + (tid % 8) * 4;
  lf32x4 acc = dM_in ? *reinterpret_cast<const lf32x4*>(dM_in + bk * D * D + eoff) : lf32x4{};
  float zacc = (do_z && tid < T && dz_in) ? dz_in[bk * D + a0 + tid] : 0.f;
  for (int sl = nseg - 1; sl >= 0; --sl) {
    const size_t unit = bk * nseg + sl;
    *reinterpret_cast<lf32x4*>(dMsnap + unit * D * D + eoff) = acc;
    acc += *reinterpret_cast<const lf32x4*>(R + unit * D * D + eoff);
    if (do_z && tid < T) {
      dzsnap[unit * D + a0 + tid] = zacc;
      zacc += r[unit * D + a0 + tid];
    }
  }
  if (dM_out) {
    *reinterpret_cast<lf32x4*>(dM_out + bk * D * D + eoff) = acc;
    if (do_z && tid < T) dz_out[bk * D + a0 + tid] = zacc;
  }
}

hipError_t launch_rscan_mfma(const Geometry& g, const void* Q, const BwdChunkWs& w, float* R, float* r,
                             const float* dM_in, const float* dz_in, float* dM_out, float* dz_out,
                             int s_begin, int s_end, hipStream_t st) {
  if (!bwd_long_mfma_supported(g)) return hipErrorInvalidValue;
  const int nseg = s_end - s_begin;
  const long long units = (long long)g.B * g.Hkv * nseg;
  if (units > 0x7fffffffLL) return hipErrorInvalidValue;
  const __bf16* q = static_cast<const __bf16*>(Q);
  if (g.D == 128)
    hipLaunchKernelGGL(rdelta_mfma_kernel<128>, dim3((unsigned)units), dim3(256), 0, st, q, w.dnum, w.dden, R, r,
                       g.Hq, g.Hkv, g.N, g.L, s_begin, nseg, g.lens);
  else
    hipLaunchKernelGGL(rdelta_mfma_kernel<64>, dim3((unsigned)units), dim3(256), 0, st, q, w.dnum, w.dden, R, r,
                       g.Hq, g.Hkv, g.N, g.L, s_begin, nseg, g.lens);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int tiles = (g.D / 32) * (g.D / 32);
  if (g.D == 128)
    hipLaunchKernelGGL(rscan_rev_kernel<128>, dim3(tiles, g.B * g.Hkv), dim3(256), 0, st, R, r, dM_in, dz_in,
                       dM_out, dz_out, w.dMsnap, w.dzsnap, nseg);
  else
    hipLaunchKernelGGL(rscan_rev_kernel<64>, dim3(tiles, g.B * g.Hkv), dim3(256), 0, st, R, r, dM_in, dz_in,
                       dM_out, dz_out, w.dMsnap, w.dzsnap, nseg);
  return hipGetLastError();
}

bool bwd_long_mfma_supported(const Geometry& g) {
  return g.fmap == 0 && g.dtype == 1 && (g.D == 64 || g.D == 128);
}

int bwd_q_mfma_row_blocks(const Geometry& g) {
  const int bm = BqCfg<64>::BM;
  static_assert(BqCfg<64>::BM == BqCfg<128>::BM, "one row-block count for both head dims");
  return (g.L + bm - 1) / bm;
}

template <int D>
static hipError_t bwd_q_mfma_t(const Geometry& g, const void* Q, const void* K, const void* V,
                               const float* beta, const void* MhiT, const void* MloT, const float* zsnap,
                               const void* dO, void* dQ, const BwdChunkWs& w, const float* lse_in, int s_begin,
                               int s_end, hipStream_t st) {
  const int nseg = s_end - s_begin;
  const float scale = 1.f / sqrtf((float)D);
  const int nqt = (g.L + BqCfg<D>::BM - 1) / BqCfg<D>::BM;
  const long long units = (long long)((nqt + 1) / 2) * g.Hq * g.B * nseg;
  if (units > 0x7fffffffLL) return hipErrorInvalidValue;
  dim3 grid((unsigned)units);
  hipLaunchKernelGGL((bwd_q_mfma_kernel<D>), grid, dim3(BqCfg<D>::NT), 0, st,
                     static_cast<const __bf16*>(Q), static_cast<const __bf16*>(K),
                     static_cast<const __bf16*>(V), beta, static_cast<const __bf16*>(MhiT),
                     static_cast<const __bf16*>(MloT), zsnap, static_cast<const __bf16*>(dO),
                     static_cast<__bf16*>(dQ), w.lse, w.Dd, w.dden, w.dnum, w.dbeta_part, lse_in, g.Hq,
                     g.Hkv, g.N, g.L, s_begin, nseg, nqt, 1.4426950408889634f * scale, scale, g.lens);
  return hipGetLastError();
}

template <int D>
static hipError_t bwd_kv_mfma_t(const Geometry& g, const void* Q, const void* K, const void* V,
                                const float* beta, const void* dO, const BwdChunkWs& w, void* dK, void* dV,
                                int s_begin, int s_end, hipStream_t st) {
  const int nseg = s_end - s_begin;
  const float scale = 1.f / sqrtf((float)D);
  const long long units = (long long)((g.L + BkCfg<D>::BK - 1) / BkCfg<D>::BK) * g.Hkv * g.B * nseg;
  if (units > 0x7fffffffLL) return hipErrorInvalidValue;
  dim3 grid((unsigned)units);
  hipLaunchKernelGGL((bwd_kv_mfma_kernel<D>), grid, dim3(BkCfg<D>::NT), 0, st,
                     static_cast<const __bf16*>(Q), static_cast<const __bf16*>(K),
                     static_cast<const __bf16*>(V), beta, static_cast<const __bf16*>(dO), w.lse, w.Dd,
                     w.dMsnap, w.dzsnap, static_cast<__bf16*>(dK), static_cast<__bf16*>(dV), g.Hq, g.Hkv,
                     g.N, g.L, s_begin, nseg, 1.4426950408889634f * scale, scale, g.lens);
  return hipGetLastError();
}

hipError_t launch_bwd_kv_mfma(const Geometry& g, const void* Q, const void* K, const void* V,
                              const float* beta, const void* dO, const BwdChunkWs& w, void* dK, void* dV,
                              int s_begin, int s_end, hipStream_t st) {
  if (!bwd_long_mfma_supported(g)) return hipErrorInvalidValue;
  if (g.D == 128) return bwd_kv_mfma_t<128>(g, Q, K, V, beta, dO, w, dK, dV, s_begin, s_end, st);
  return bwd_kv_mfma_t<64>(g, Q, K, V, beta, dO, w, dK, dV, s_begin, s_end, st);
}

hipError_t launch_bwd_q_mfma(const Geometry& g, const void* Q, const void* K, const void* V,
                             const float* beta, const void* MhiT, const void* MloT, const float* zsnap,
                             const void* dO, void* dQ, const BwdChunkWs& w, const float* lse_in, int s_begin,
                             int s_end, hipStream_t st) {
  if (!bwd_long_mfma_supported(g)) return hipErrorInvalidValue;
  if (g.D == 128) return bwd_q_mfma_t<128>(g, Q, K, V, beta, MhiT, MloT, zsnap, dO, dQ, w, lse_in, s_begin, s_end, st);
  return bwd_q_mfma_t<64>(g, Q, K, V, beta, MhiT, MloT, zsnap, dO, dQ, w, lse_in, s_begin, s_end, st);
}

}  // namespace infini
