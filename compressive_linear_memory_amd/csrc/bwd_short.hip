// Fused backward for short segments (seg_len <= 64, bf16, head_dim 64 or 128).
//
// The exact derivative of the forward (page "Hugging Face Infini-Attention
// 재현 분석", section "Infini-Attention 메커니즘"), for
// loss = <dO, O> + <dM_S, M_S> + <dz_S, z_S>.  One workgroup per (batch, K/V
// head):
//   1. replays the memory path forward, M += sigma(K)^T V, to reach M_S
//      (the state lives in v_mfma_f32_16x16x32_bf16 accumulators);
//   2. walks the segments from last to first holding M and dM = dL/dM_s in
//      accumulators.  At segment s > 0 it first recovers M_{s-1} = M_s -
//      sigma(K_s)^T V_s by subtracting exactly the bf16 products the replay
//      added (segment 0 reloads the state passed in, so that an empty memory,
//      whose retrieval denominator is eps alone, stays exactly empty), then
//        update backward:  dV += sigma(K) dM, dK += (V dM^T + dz) * sigma'(K)
//        per query head:   recompute P (exact softmax, the whole segment is one
//                          tile), A_dot, A_mem; gate gradients;
//                          dnum = g dO / den, dden = -rowsum(g dO * A_mem) / den,
//                          dQ = (dnum M^T + dden z^T) * sigma'(Q) + dS K / sqrt d,
//                          dS = P * (dA_dot V^T - rowsum(dA_dot * A_dot)),
//                          dK += dS^T Q / sqrt d, dV += P^T dA_dot,
//                          dM += sigma(Q)^T dnum, dz += sigma(Q)^T dden
//      (the retrieval terms are added after the update backward has used dM,
//      so dM then holds dL/dM_{s-1}).
//   dbeta = g(1-g) sum dO * (A_mem - A_dot) is summed per head in fp32 from
//   the recomputed A_mem and A_dot and finished by dbeta_finish_kernel.
//
// Operands whose contraction index runs along LDS rows are read with the
// gfx950 transpose load ds_read_b64_tr_b16: in each group of 16 lanes, lane j
// receives element j%4 of the 4-element chunks addressed by lanes j/4,
// j/4+4, j/4+8, j/4+12.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace infini {

typedef __bf16 bbf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bbf16x4 __attribute__((ext_vector_type(4)));
typedef short bs16x4 __attribute__((ext_vector_type(4)));
typedef float bf32x4 __attribute__((ext_vector_type(4)));

constexpr int kBwdMaxGroup = 16;   // query heads per K/V head handled by the fused kernel

template <int D>
struct BwdCfg {
  static constexpr int BL = 64;
  static constexpr int KS = D / 32;       // k-steps over head_dim
  static constexpr int DB = D / 16;       // 16-blocks of head_dim
  static constexpr int AB = DB / 4;       // state row blocks per wave
  static constexpr int RS = D + 8;        // row stride of [64][D] and [D][D] tiles
  static constexpr int PS = BL + 8;       // row stride of [64][64] tiles
  static constexpr int KPT = D / 32;      // keys per thread in staging
  static constexpr int NKG = BL / KPT;
};

__device__ __forceinline__ bbf16x4 tr4(const __bf16* p) {
  const bs16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) bs16x4*)(p));
  return __builtin_bit_cast(bbf16x4, v);
}

// Operand for row r0 + lane%16 of X^T where X is stored row-major X[k][r]
// (row stride xs): element e of the result is X[k0 + e][.] for e < 4 and
// X[k1 + e - 4][.] for e >= 4 (k0, k1 may differ per lane group).
__device__ __forceinline__ bbf16x8 tr_op(const __bf16* X, int xs, int r0, int k0, int k1, int lane) {
  const int i = lane & 15;
  const int e = i >> 2, a = i & 3;
  const bbf16x4 lo = tr4(X + (k0 + e) * xs + r0 + 4 * a);
  const bbf16x4 hi = tr4(X + (k1 + e) * xs + r0 + 4 * a);
  return bbf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ bbf16x8 sigma8(bbf16x8 x) {
  bbf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)elu1((float)x[e]);
  return r;
}

__device__ __forceinline__ float red16x4(float x) {     // sum over the 4 lane groups of 16
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

template <int D>
__global__ __launch_bounds__(256)
void bwd_short_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                      const __bf16* __restrict__ V, const float* __restrict__ beta,
                      const float* __restrict__ M0, const float* __restrict__ z0,
                      const __bf16* __restrict__ dO, const float* __restrict__ dM_S,
                      const float* __restrict__ dz_S, __bf16* __restrict__ dQ,
                      __bf16* __restrict__ dK, __bf16* __restrict__ dV,
                      float* __restrict__ dM0, float* __restrict__ dz0,
                      float* __restrict__ dbeta_part, const float* __restrict__ lse,
                      const int* __restrict__ lens, const float* __restrict__ Ms_in,
                      const float* __restrict__ zs_in, int Hq, int Hkv, int N, int L, float scale, float sl2) {
  using C = BwdCfg<D>;
  constexpr int RS = C::RS, PS = C::PS;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[C::BL * RS];
  __shared__ __attribute__((aligned(16))) __bf16 Vr[C::BL * RS];
  __shared__ __attribute__((aligned(16))) __bf16 Mt[D * RS];    // M_{s-1}^T  [c][a]
  __shared__ __attribute__((aligned(16))) __bf16 dMt[D * RS];   // dM^T [c][a], then low part of M^T
  __shared__ __attribute__((aligned(16))) __bf16 Qs[C::BL * RS];
  __shared__ __attribute__((aligned(16))) __bf16 Xb[C::BL * RS];   // dA_dot, then dnum, rows q
  __shared__ __attribute__((aligned(16))) __bf16 Pb[C::BL * PS];   // P rows q
  __shared__ __attribute__((aligned(16))) __bf16 Sb[C::BL * PS];   // dS rows q
  __shared__ __attribute__((aligned(16))) float zs[D];
  __shared__ float dzs[D];
  __shared__ __attribute__((aligned(16))) float dds[C::BL];
  __shared__ float dbacc[kBwdMaxGroup][4];

  const int bk = blockIdx.x;
  const int b = bk / Hkv, kvh = bk % Hkv;
  const int G = Hq / Hkv;
  const int Nb = seq_len_of(lens, b, N);    // tokens of this sequence
  const int S = (Nb + L - 1) / L;           // the last segment may be short
  // Lane indices.  They are passed through an empty asm statement at the
  // top of each segment and head step ("refresh"), so that the compiler
  // recomputes the addresses derived from them there instead of keeping
  // dozens of them live (and spilled) across the whole loop.
  int tid = threadIdx.x;
  int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int lc = lane & 15, g = lane >> 4;
  const size_t kvbase = ((size_t)b * Hkv + kvh) * N * D;

  // ---- resident state: M and dM blocks (a = ab*16 + 4g + i, c = cb*16 + lc)
  bf32x4 macc[C::AB][C::DB], dmacc[C::AB][C::DB];
  bf32x4 zacc[C::AB];                      // z rows a = ab*16 + 4g + i (every column lc alike)
#pragma unroll
  for (int x = 0; x < C::AB; ++x)
#pragma unroll
    for (int cb = 0; cb < C::DB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const size_t off = (size_t)bk * D * D + (size_t)((wave * C::AB + x) * 16 + 4 * g + i) * D + cb * 16 + lc;
        // the walk back starts from M_S: the forward's, when given, else
        // M0 plus the replay below
        macc[x][cb][i] = Ms_in ? Ms_in[off] : M0 ? M0[off] : 0.f;
        dmacc[x][cb][i] = dM_S ? dM_S[off] : 0.f;
      }
#pragma unroll
  for (int x = 0; x < C::AB; ++x)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t off = (size_t)bk * D + (wave * C::AB + x) * 16 + 4 * g + i;
      zacc[x][i] = zs_in ? zs_in[off] : z0 ? z0[off] : 0.f;
    }
  for (int a = tid; a < D; a += 256) dzs[a] = dz_S ? dz_S[(size_t)bk * D + a] : 0.f;
  if (tid < kBwdMaxGroup * 4) dbacc[tid / 4][tid % 4] = 0.f;

  // ---- staging of segment s: K and V rows (V rows past the end are zero).
  // The rows are loaded into registers one segment ahead (load_kv) and
  // written to LDS when the segment starts (store_kv), so the load latency
  // hides behind the previous segment's work.
  int kg = tid % C::NKG, dc = tid / C::NKG;
  bbf16x8 kst[C::KPT], vst[C::KPT];
  auto load_kv = [&](int s) {
    const int Lk = min(L, Nb - s * L);     // keys of this segment
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const size_t off = kvbase + ((size_t)s * L + min(kg * C::KPT + i, Lk - 1)) * D + dc * 8;
      kst[i] = *reinterpret_cast<const bbf16x8*>(K + off);
      vst[i] = *reinterpret_cast<const bbf16x8*>(V + off);
    }
  };
  auto store_kv = [&](int s) {
    const int Lk = min(L, Nb - s * L);
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int key = kg * C::KPT + i;
      const bool in = key < Lk;
      *reinterpret_cast<bbf16x8*>(Ks + key * RS + dc * 8) = kst[i];
      *reinterpret_cast<bbf16x8*>(Vr + key * RS + dc * 8) = in ? vst[i] : bbf16x8{};
    }
  };
  // M +=/-= sigma(K)^T V and z +=/-= sigma(K)^T 1 from the staged tiles (keys
  // 32t + 8g + e; keys past the segment end, Lk and on, contribute zero): the
  // same bf16 products, in the same order, as the forward's update, so that
  // the state replayed here is the forward's and subtracting recovers the
  // earlier one step by step
  const bbf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                        (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
  auto state_update = [&](bool subtract, int Lk) {
#pragma unroll
    for (int x = 0; x < C::AB; ++x) {
      const int ab = wave * C::AB + x;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bbf16x8 a = sigma8(tr_op(Ks, RS, ab * 16, 32 * t + 8 * g, 32 * t + 8 * g + 4, lane));
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (32 * t + 8 * g + e >= Lk) a[e] = (__bf16)0.f;
        if (subtract) {   // flip the bf16 sign bits
          typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
          u32x4 u = __builtin_bit_cast(u32x4, a);
          u ^= 0x80008000u;
          a = __builtin_bit_cast(bbf16x8, u);
        }
        zacc[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ones, zacc[x], 0, 0, 0);
#pragma unroll
        for (int cb = 0; cb < C::DB; ++cb) {
          const bbf16x8 bb = tr_op(Vr, RS, cb * 16, 32 * t + 8 * g, 32 * t + 8 * g + 4, lane);
          macc[x][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb, macc[x][cb], 0, 0, 0);
        }
      }
    }
  };
  // state blocks -> bf16 transposed tile [c][a] (lane holds 4 consecutive a)
  auto publish = [&](bf32x4 (&acc)[C::AB][C::DB], __bf16* T) {
#pragma unroll
    for (int x = 0; x < C::AB; ++x)
#pragma unroll
      for (int cb = 0; cb < C::DB; ++cb)
        *reinterpret_cast<bbf16x4*>(T + (cb * 16 + lc) * RS + (wave * C::AB + x) * 16 + 4 * g) =
            bbf16x4{(__bf16)acc[x][cb][0], (__bf16)acc[x][cb][1], (__bf16)acc[x][cb][2], (__bf16)acc[x][cb][3]};
  };

  // ---- 1. replay the memory path to M_S, z_S (unless the forward's was given)
  const int Sr = Ms_in ? 0 : S;
  if (S > 0) load_kv(Sr > 0 ? 0 : S - 1);
  for (int s = 0; s < Sr; ++s) {
    store_kv(s);
    load_kv(min(s + 1, S - 1));            // the last one is segment S-1 again: phase 2 starts there
    lds_barrier();
    state_update(false, min(L, Nb - s * L));
    lds_barrier();
  }

  int q = wave * 16 + lc;                  // query row of this lane (query-side products)
  int jk = wave * 16 + lc;                 // key row of this lane (key-side products)
  auto refresh = [&]() {
    asm volatile("" : "+v"(tid), "+v"(lane), "+v"(lc), "+v"(g), "+v"(kg), "+v"(dc), "+v"(q), "+v"(jk));
  };

  // Q rows and this lane's dO pieces of a head (the Q rows are staged into
  // LDS per head step); those of the group's first head are loaded at the
  // start of the segment, so that they arrive during the state recovery and
  // the update backward
  constexpr int QPT = C::BL * D / 8 / 256;
  bbf16x8 qpre[QPT];
  bbf16x4 dpre[C::DB];
  auto load_qdo = [&](int s, int h) {
    const int Lq = min(L, Nb - s * L);
    const size_t qb = (((size_t)b * Hq + h) * N + (size_t)s * L) * D;
    const __bf16* dop = dO + qb + (size_t)min(q, Lq - 1) * D;
#pragma unroll
    for (int cb = 0; cb < C::DB; ++cb) dpre[cb] = *reinterpret_cast<const bbf16x4*>(dop + cb * 16 + 4 * g);
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int c = tid + i * 256, row = c / (D / 8), col = (c % (D / 8)) * 8;
      qpre[i] = *reinterpret_cast<const bbf16x8*>(Q + qb + (size_t)min(row, Lq - 1) * D + col);
    }
  };

  // ---- 2. segments in reverse
  for (int s = S - 1; s >= 0; --s) {
    refresh();
    const int Ls = min(L, Nb - s * L);     // rows and keys of this segment
    if (s == 0) {
      // M_{-1}, z_{-1}: the state passed in, exactly (an empty memory must
      // stay exactly empty: its retrieval denominator is eps alone).  Read
      // before the segment's own loads are issued, so that waiting for it
      // does not wait for them.
#pragma unroll
      for (int x = 0; x < C::AB; ++x)
#pragma unroll
        for (int cb = 0; cb < C::DB; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            macc[x][cb][i] = M0 ? M0[(size_t)bk * D * D + (size_t)((wave * C::AB + x) * 16 + 4 * g + i) * D + cb * 16 + lc] : 0.f;
#pragma unroll
      for (int x = 0; x < C::AB; ++x)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          zacc[x][i] = z0 ? z0[(size_t)bk * D + (wave * C::AB + x) * 16 + 4 * g + i] : 0.f;
    }
    load_qdo(s, kvh * G);                  // the first head's rows
    store_kv(s);
    lds_barrier();
    if (s > 0) state_update(true, Ls);     // M_{s-1}, z_{s-1}
    publish(macc, Mt);
    publish(dmacc, dMt);
#pragma unroll
    for (int x = 0; x < C::AB; ++x)
      if (lc == 0) *reinterpret_cast<bf32x4*>(zs + (wave * C::AB + x) * 16 + 4 * g) = zacc[x];
    lds_barrier();

    // update backward (key-side: this wave's 16 keys), with dM = dL/dM_s
    bf32x4 dkacc[C::DB], dvacc[C::DB];
#pragma unroll
    for (int ab = 0; ab < C::DB; ++ab) {
      // (dM V^T)[a][j]: A = dM rows a (k = c), B = V[j][c]
      bf32x4 acc = {};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bbf16x8 a = tr_op(dMt, RS, ab * 16, 32 * ks + 8 * g, 32 * ks + 8 * g + 4, lane);
        const bbf16x8 bb = *reinterpret_cast<const bbf16x8*>(Vr + jk * RS + 32 * ks + 8 * g);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb, acc, 0, 0, 0);
      }
      const bbf16x4 kv = *reinterpret_cast<const bbf16x4*>(Ks + jk * RS + ab * 16 + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = (acc[i] + dzs[ab * 16 + 4 * g + i]) * elu1_grad((float)kv[i]);
      dkacc[ab] = acc;
    }
    bbf16x8 skr[C::KS];                    // sigma(K) of this lane's key row, k = 32 ks + 8g ..
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) skr[ks] = sigma8(*reinterpret_cast<const bbf16x8*>(Ks + jk * RS + 32 * ks + 8 * g));
#pragma unroll
    for (int cb = 0; cb < C::DB; ++cb) {
      // (dM^T sigma(K)^T)[c][j]: A = dM^T rows c (k = a), B = sigma(K)[j][a]
      bf32x4 acc = {};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bbf16x8 a = *reinterpret_cast<const bbf16x8*>(dMt + (cb * 16 + lc) * RS + 32 * ks + 8 * g);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, skr[ks], acc, 0, 0, 0);
      }
      dvacc[cb] = acc;
    }

    // The retrieval gradient dnum M^T + dden z^T is a difference of two
    // nearly equal terms, so M enters it (and A_mem) as a bf16 hi/lo pair:
    // the low part M - bf16(M) replaces dM^T, which the update backward has
    // finished with.
    lds_barrier();
#pragma unroll
    for (int x = 0; x < C::AB; ++x)
#pragma unroll
      for (int cb = 0; cb < C::DB; ++cb) {
        bbf16x4 lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) lo[i] = (__bf16)(macc[x][cb][i] - (float)(__bf16)macc[x][cb][i]);
        *reinterpret_cast<bbf16x4*>(dMt + (cb * 16 + lc) * RS + (wave * C::AB + x) * 16 + 4 * g) = lo;
      }
    const __bf16* Mlo = dMt;

    // one query head of the group; the last one also issues the loads of the
    // next segment's K and V rows (a separate inlined copy, so that those
    // registers are live only from there on)
    auto head_step = [&](const int h, const bool prefetch) {
      refresh();
      // register classes: the state, its gradient and the dK / dV
      // accumulators are read only by the matrix cores inside this loop
#pragma unroll
      for (int x = 0; x < C::AB; ++x)
#pragma unroll
        for (int cb = 0; cb < C::DB; ++cb) {
          asm volatile("" : "+a"(macc[x][cb]));
          asm volatile("" : "+a"(dmacc[x][cb]));
        }
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        asm volatile("" : "+a"(dkacc[db]));
        asm volatile("" : "+a"(dvacc[db]));
      }
      const size_t qb = (((size_t)b * Hq + h) * N + (size_t)s * L) * D;
      // this lane's dO pieces (row q, columns cb*16 + 4g ..) are used after
      // the score and retrieval products; the Q rows are staged now
      if (h != kvh * G) load_qdo(s, h);
      bbf16x4 dov[C::DB];
#pragma unroll
      for (int cb = 0; cb < C::DB; ++cb) dov[cb] = dpre[cb];
#pragma unroll
      for (int i = 0; i < QPT; ++i) {
        const int c = tid + i * 256, row = c / (D / 8), col = (c % (D / 8)) * 8;
        *reinterpret_cast<bbf16x8*>(Qs + row * RS + col) = qpre[i];
      }
      lds_barrier();

      const bool qok = q < Ls;
      const float gt = sigmoid(beta[h]);
      bbf16x8 qreg[C::KS];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) qreg[ks] = *reinterpret_cast<const bbf16x8*>(Qs + q * RS + 32 * ks + 8 * g);
      // S^T = K Q^T; element (kb, i) is key 16kb + 4g + i
      bf32x4 pacc[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        pacc[kb] = bf32x4{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const bbf16x8 a = *reinterpret_cast<const bbf16x8*>(Ks + (kb * 16 + lc) * RS + 32 * ks + 8 * g);
          pacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[ks], pacc[kb], 0, 0, 0);
        }
      }
      const int lim = min(q, Ls - 1);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb * 16 + 4 * g + i > lim) pacc[kb][i] = -INFINITY;
      // With the forward's row log-sum-exp the probabilities come out
      // normalised (1/l = 1); otherwise they are formed against the row max
      // and normalised by their own sum.
      float mref;
      if (lse) {
        mref = lse[((size_t)b * Hq + h) * N + (size_t)s * L + lim] * 1.4426950408889634f;
      } else {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, pacc[kb][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        mref = mx * sl2;
      }
      float lsum = 0.f;
      bbf16x8 pb[2];     // P^T operand, slot 8g + x <-> key 32t + 16(x/4) + 4g + x%4
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const __bf16 pr = (__bf16)__builtin_amdgcn_exp2f(fmaf(pacc[kb][i], sl2, -mref));
          lsum += (float)pr;
          pb[kb >> 1][(kb & 1) * 4 + i] = pr;
        }
      const float inv_l = lse ? 1.f : 1.f / red16x4(lsum);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) pacc[kb][i] = (float)pb[kb >> 1][(kb & 1) * 4 + i] * inv_l;   // P
      // A_dot^T = V^T P^T (unnormalised)
      bf32x4 oacc[C::DB];
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        oacc[db] = bf32x4{};
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bbf16x8 a = tr_op(Vr, RS, db * 16, 32 * t + 4 * g, 32 * t + 16 + 4 * g, lane);
          oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[t], oacc[db], 0, 0, 0);
        }
      }
      // den = sigma(Q) z_{s-1} + eps
      bbf16x8 sq[C::KS];
      float dpart = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        sq[ks] = sigma8(qreg[ks]);
#pragma unroll
        for (int e = 0; e < 8; ++e) dpart += (float)sq[ks][e] * zs[32 * ks + 8 * g + e];
      }
      const float den = red16x4(dpart) + 1e-6f;
      const float inv_den = 1.f / den;
      // gate and retrieval gradients per (q, c = cb*16 + 4g + i)
      float bsum = 0.f, ddot = 0.f, dmem = 0.f;
      bbf16x8 dnp[C::KS], dap[C::KS];     // dnum, dA_dot packed like pb (c in place of keys)
#pragma unroll
      for (int cb = 0; cb < C::DB; ++cb) {
        bf32x4 nacc = {};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const bbf16x8 a = *reinterpret_cast<const bbf16x8*>(Mt + (cb * 16 + lc) * RS + 32 * ks + 8 * g);
          const bbf16x8 al = *reinterpret_cast<const bbf16x8*>(Mlo + (cb * 16 + lc) * RS + 32 * ks + 8 * g);
          nacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, sq[ks], nacc, 0, 0, 0);
          nacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, sq[ks], nacc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float go = qok ? (float)dov[cb][i] : 0.f;
          const float am = nacc[i] * inv_den;
          const float ad = oacc[cb][i] * inv_l;
          // the row sums pair with the rounded operands the products use, so
          // that dP - Dd and dnum M^T + dden z^T cancel as they do exactly
          const __bf16 dn = (__bf16)(gt * go * inv_den);
          const __bf16 da = (__bf16)((1.f - gt) * go);
          bsum += go * (am - ad);
          ddot += (float)da * ad;
          dmem += (float)dn * am;
          dnp[cb >> 1][(cb & 1) * 4 + i] = dn;
          dap[cb >> 1][(cb & 1) * 4 + i] = da;
        }
      }
      const float Dd = red16x4(ddot);                        // rowsum(dA_dot * A_dot)
      const float dden = -red16x4(dmem);
      bsum = wave_sum(bsum);                                 // this wave's 16 query rows
      // dP^T = V dA_dot^T; dS = P (dP - Dd)
      bbf16x8 dsp[2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        bf32x4 acc = {};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const __bf16* vp = Vr + (kb * 16 + lc) * RS + 32 * ks + 4 * g;
          const bbf16x4 lo = *reinterpret_cast<const bbf16x4*>(vp);
          const bbf16x4 hi = *reinterpret_cast<const bbf16x4*>(vp + 16);
          const bbf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, dap[ks], acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) dsp[kb >> 1][(kb & 1) * 4 + i] = (__bf16)(scale * pacc[kb][i] * (acc[i] - Dd));
      }
      // dQ per 16 columns a: (dnum M^T + dden z) sigma'(Q) + scale dS K
      __bf16* dqp = dQ + qb + (size_t)q * D;
#pragma unroll
      for (int ab = 0; ab < C::DB; ++ab) {
        bf32x4 ret = {}, loc = {};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const bbf16x8 a = tr_op(Mt, RS, ab * 16, 32 * ks + 4 * g, 32 * ks + 16 + 4 * g, lane);
          const bbf16x8 al = tr_op(Mlo, RS, ab * 16, 32 * ks + 4 * g, 32 * ks + 16 + 4 * g, lane);
          ret = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, dnp[ks], ret, 0, 0, 0);
          ret = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, dnp[ks], ret, 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bbf16x8 a = tr_op(Ks, RS, ab * 16, 32 * t + 4 * g, 32 * t + 16 + 4 * g, lane);
          loc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, dsp[t], loc, 0, 0, 0);
        }
        const bbf16x4 qv = *reinterpret_cast<const bbf16x4*>(Qs + q * RS + ab * 16 + 4 * g);
        if (qok) {
          bbf16x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            w[i] = (__bf16)((ret[i] + dden * zs[ab * 16 + 4 * g + i]) * elu1_grad((float)qv[i]) + loc[i]);
          *reinterpret_cast<bbf16x4*>(dqp + ab * 16 + 4 * g) = w;
        }
      }
      // rows for the key-side products: P (unnormalised bf16), dS; dden
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        *reinterpret_cast<bbf16x4*>(Pb + q * PS + 32 * t + 4 * g) = bbf16x4{pb[t][0], pb[t][1], pb[t][2], pb[t][3]};
        *reinterpret_cast<bbf16x4*>(Pb + q * PS + 32 * t + 16 + 4 * g) = bbf16x4{pb[t][4], pb[t][5], pb[t][6], pb[t][7]};
        *reinterpret_cast<bbf16x4*>(Sb + q * PS + 32 * t + 4 * g) = bbf16x4{dsp[t][0], dsp[t][1], dsp[t][2], dsp[t][3]};
        *reinterpret_cast<bbf16x4*>(Sb + q * PS + 32 * t + 16 + 4 * g) = bbf16x4{dsp[t][4], dsp[t][5], dsp[t][6], dsp[t][7]};
      }
      if (prefetch) load_kv(s - 1);       // the next segment's rows
      if (g == 0) dds[q] = qok ? dden : 0.f;
      if (lane == 0) dbacc[h - kvh * G][wave] += bsum;   // each wave owns its slot: fixed order
      lds_barrier();
      // key side, contracting over the segment's queries: dK^T += Q^T dS
      // (dS carries the softmax scale)
#pragma unroll
      for (int ab = 0; ab < C::DB; ++ab) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bbf16x8 a = tr_op(Qs, RS, ab * 16, 32 * t + 8 * g, 32 * t + 8 * g + 4, lane);
          const bbf16x8 bb = tr_op(Sb, PS, wave * 16, 32 * t + 8 * g, 32 * t + 8 * g + 4, lane);
          dkacc[ab] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb, dkacc[ab], 0, 0, 0);
        }
      }
      // Xb <- dA_dot rows times 1/l of their query row: Pb holds the
      // unnormalised probabilities, so Pb^T Xb is P^T dA_dot; then dV^T += Xb^T Pb
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        bbf16x8 w;
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = (__bf16)((float)dap[ks][e] * inv_l);
        *reinterpret_cast<bbf16x4*>(Xb + q * RS + 32 * ks + 4 * g) = bbf16x4{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<bbf16x4*>(Xb + q * RS + 32 * ks + 16 + 4 * g) = bbf16x4{w[4], w[5], w[6], w[7]};
      }
      lds_barrier();
#pragma unroll
      for (int cb = 0; cb < C::DB; ++cb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bbf16x8 a = tr_op(Xb, RS, cb * 16, 32 * t + 8 * g, 32 * t + 8 * g + 4, lane);
          const bbf16x8 bb = tr_op(Pb, PS, wave * 16, 32 * t + 8 * g, 32 * t + 8 * g + 4, lane);
          dvacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb, dvacc[cb], 0, 0, 0);
        }
      }
      lds_barrier();
      // Xb <- dnum rows; dM += sigma(Q)^T dnum, dz += sigma(Q)^T dden
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        *reinterpret_cast<bbf16x4*>(Xb + q * RS + 32 * ks + 4 * g) = bbf16x4{dnp[ks][0], dnp[ks][1], dnp[ks][2], dnp[ks][3]};
        *reinterpret_cast<bbf16x4*>(Xb + q * RS + 32 * ks + 16 + 4 * g) = bbf16x4{dnp[ks][4], dnp[ks][5], dnp[ks][6], dnp[ks][7]};
      }
      lds_barrier();
#pragma unroll
      for (int x = 0; x < C::AB; ++x) {
        const int ab = wave * C::AB + x;
        float zp = 0.f;                    // dz of row a = ab*16 + lc over this lane's 16 queries
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          bbf16x8 a = tr_op(Qs, RS, ab * 16, 32 * t + 8 * g, 32 * t + 8 * g + 4, lane);
          a = sigma8(a);
          // query rows past the segment end carry zero dnum and zero dden
#pragma unroll
          for (int cb = 0; cb < C::DB; ++cb) {
            const bbf16x8 bb = tr_op(Xb, RS, cb * 16, 32 * t + 8 * g, 32 * t + 8 * g + 4, lane);
            dmacc[x][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb, dmacc[x][cb], 0, 0, 0);
          }
          const bf32x4 d0 = *reinterpret_cast<const bf32x4*>(dds + 32 * t + 8 * g);
          const bf32x4 d1 = *reinterpret_cast<const bf32x4*>(dds + 32 * t + 8 * g + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) zp += (float)a[e] * d0[e] + (float)a[e + 4] * d1[e];
        }
        zp = red16x4(zp);
        if (g == 0) dzs[ab * 16 + lc] += zp;   // each wave owns its rows
      }
      lds_barrier();
    };
    for (int h = kvh * G; h < (kvh + 1) * G - 1; ++h) head_step(h, false);
    head_step((kvh + 1) * G - 1, s > 0);

    // dK, dV of this segment's keys.  Each wave passes its 16 rows through
    // LDS (rows of Xb and Qs, free here; every other wave is done with them,
    // and the next writes come after the next segment's first barrier), so
    // that the global stores are whole 16-byte row pieces, 1 KB per
    // instruction, instead of 32-byte pieces of 16 rows
    refresh();
    {
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        *reinterpret_cast<bbf16x4*>(Xb + jk * RS + db * 16 + 4 * g) =
            bbf16x4{(__bf16)dkacc[db][0], (__bf16)dkacc[db][1], (__bf16)dkacc[db][2], (__bf16)dkacc[db][3]};
        *reinterpret_cast<bbf16x4*>(Qs + jk * RS + db * 16 + 4 * g) =
            bbf16x4{(__bf16)dvacc[db][0], (__bf16)dvacc[db][1], (__bf16)dvacc[db][2], (__bf16)dvacc[db][3]};
      }
      // the wave reads back rows other lanes of it wrote (LDS is in order
      // within a wave; the fences keep the compiler from reordering)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
      constexpr int CPR = D / 8;                   // 16-byte pieces per row
#pragma unroll
      for (int i = 0; i < 16 * CPR / 64; ++i) {
        const int c = lane + 64 * i, key = wave * 16 + c / CPR, col = (c % CPR) * 8;
        if (key < Ls) {
          const size_t kr = kvbase + ((size_t)s * L + key) * D + col;
          *reinterpret_cast<bbf16x8*>(dK + kr) = *reinterpret_cast<const bbf16x8*>(Xb + key * RS + col);
          *reinterpret_cast<bbf16x8*>(dV + kr) = *reinterpret_cast<const bbf16x8*>(Qs + key * RS + col);
        }
      }
    }
  }

  if (dM0) {
#pragma unroll
    for (int x = 0; x < C::AB; ++x)
#pragma unroll
      for (int cb = 0; cb < C::DB; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dM0[(size_t)bk * D * D + (size_t)((wave * C::AB + x) * 16 + 4 * g + i) * D + cb * 16 + lc] = dmacc[x][cb][i];
    for (int a = tid; a < D; a += 256) dz0[(size_t)bk * D + a] = dzs[a];
  }
  if (tid < G) dbeta_part[(size_t)b * Hq + kvh * G + tid] =
      ((dbacc[tid][0] + dbacc[tid][1]) + dbacc[tid][2]) + dbacc[tid][3];
}

__global__ void dbeta_finish_kernel(const float* __restrict__ beta, const float* __restrict__ part,
                                    float* __restrict__ dbeta, int B, int Hq) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= Hq) return;
  float t = 0.f;
  for (int b = 0; b < B; ++b) t += part[(size_t)b * Hq + h];
  const float gt = sigmoid(beta[h]);
  dbeta[h] = gt * (1.f - gt) * t;
}

bool bwd_short_supported(const Geometry& g) {
  return g.fmap == 0 && g.dtype == 1 && (g.D == 64 || g.D == 128) && g.L <= 64 && g.G() <= kBwdMaxGroup;
}

hipError_t launch_bwd_short(const Geometry& g, const void* Q, const void* K, const void* V,
                            const float* beta, const float* M0, const float* z0, const void* dO,
                            const float* dM_S, const float* dz_S, void* dQ, void* dK, void* dV,
                            float* dbeta, float* dM0, float* dz0, float* dbeta_part, const float* lse,
                            hipStream_t st, const float* M_S_in, const float* z_S_in) {
  if (!bwd_short_supported(g)) return hipErrorInvalidValue;
  const float scale = 1.f / sqrtf((float)g.D);
  const float sl2 = 1.4426950408889634f * scale;
#define BS_ARGS static_cast<const __bf16*>(Q), static_cast<const __bf16*>(K), static_cast<const __bf16*>(V), beta, \
                M0, z0, static_cast<const __bf16*>(dO), dM_S, dz_S, static_cast<__bf16*>(dQ), static_cast<__bf16*>(dK), \
                static_cast<__bf16*>(dV), dM0, dz0, dbeta_part, lse, g.lens, M_S_in, z_S_in, g.Hq, g.Hkv, g.N, g.L, \
                scale, sl2
  if (g.D == 128) hipLaunchKernelGGL(bwd_short_kernel<128>, dim3(g.B * g.Hkv), dim3(256), 0, st, BS_ARGS);
  else hipLaunchKernelGGL(bwd_short_kernel<64>, dim3(g.B * g.Hkv), dim3(256), 0, st, BS_ARGS);
#undef BS_ARGS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dbeta_finish_kernel, dim3((g.Hq + 63) / 64), dim3(64), 0, st, beta, dbeta_part, dbeta, g.B, g.Hq);
  return hipGetLastError();
}

}  // namespace infini
