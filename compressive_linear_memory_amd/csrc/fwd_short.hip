// Fused forward for short segments (seg_len <= 64, bf16, head_dim 64 or 128).
//
// One workgroup per (batch, K/V head) walks the segments in order with the
// memory resident on chip for the whole sequence (page "Hugging Face
// Infini-Attention 재현 분석", section "Infini-Attention 메커니즘", steps
// Segmentation to State Transfer):
//   M (fp32, d x d) lives in the accumulators of v_mfma_f32_16x16x32_bf16;
//   the update M += sigma(K)^T V is one more MFMA chain into them, and a bf16
//   transposed copy of M_{s-1} sits in LDS as the retrieval operand;
//   z (fp32, d) lives in LDS.
// Per segment (64 tokens, every query head of the group in turn): each of the
// four waves owns 16 query rows and computes S^T = K Q^T (all keys of the
// segment fit one tile, so the softmax is exact, not online), O^T = V^T P^T,
// A_mem^T = M^T sigma(Q)^T, den = sigma(Q) z + eps and the gate, then one
// bf16 store.  The next segment's K and V are loaded while this one computes.
// Nothing but (M, z) crosses segments and nothing but the final state leaves
// the chip.
//
// When few (batch, K/V head) pairs are in flight the segments of a pair are
// dealt to `parts` workgroups in consecutive ranges; part p first replays the
// memory update alone (no attention) over the segments before its range to
// reach its starting state, then processes its range fully.  A replayed
// segment costs about kReplayCost of a full one (measured at the 200M-model
// shape), so later parts get shorter ranges: part p starts at
// b_p = c (1 - (1 - r)^p) / r with c chosen so that b_parts = S, which gives
// every part the same cost.  Only the last part writes the final state.
//
// 16x16x32 bf16 operand layout (gfx950): A lane l holds row l%16, k = 8(l/16)..+7;
// B lane l holds column l%16, same k; C/D lane l holds column l%16,
// rows 4(l/16) + i, i = 0..3.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace infini {

typedef __bf16 sbf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 sbf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 sbf16x2 __attribute__((ext_vector_type(2)));
typedef float sf32x4 __attribute__((ext_vector_type(4)));

constexpr float kReplayCost = 0.45f;      // replayed segment / fully processed segment

template <int D>
struct ShortCfg {
  static constexpr int BL = 64;           // segment tile (keys and queries)
  static constexpr int KS = D / 32;       // MFMA k-steps over head_dim
  static constexpr int DB = D / 16;       // 16-row blocks of head_dim
  static constexpr int KSTR = D + 8;      // K rows (row-major)
  static constexpr int TSTR = BL + 8;     // key-contiguous rows (V^T, sigma(K)^T)
  static constexpr int MSTR = D + 8;      // M^T rows
  static constexpr int KPT = D / 32;      // keys per thread in staging (4 or 2)
  static constexpr int NKG = BL / KPT;    // key groups
  static constexpr int AB = DB / 4;       // M row blocks owned per wave
  static constexpr int KTILE = BL * KSTR;
  static constexpr int TTILE = D * TSTR;
  static constexpr int MTILE = D * MSTR;
};

template <int D>
__global__ __launch_bounds__(256)
void fwd_short_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                      const __bf16* __restrict__ V, const float* __restrict__ beta,
                      const float* __restrict__ M0, const float* __restrict__ z0,
                      __bf16* __restrict__ O, float* __restrict__ M_S, float* __restrict__ z_S,
                      float* __restrict__ lse, const int* __restrict__ lens, int Hq, int Hkv, int N, int L,
                      int parts, float sl2) {
  using C = ShortCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[C::KTILE];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[C::TTILE];
  __shared__ __attribute__((aligned(16))) __bf16 SKt[C::TTILE];
  __shared__ __attribute__((aligned(16))) __bf16 Mt[C::MTILE];
  __shared__ float zs[D];
  __shared__ float zred[C::NKG][D + 1];

  const int bk = blockIdx.x / parts;               // b * Hkv + kvh
  const int part = blockIdx.x % parts;
  const int b = bk / Hkv, kvh = bk % Hkv;
  const int G = Hq / Hkv;
  const int Nb = seq_len_of(lens, b, N);    // tokens of this sequence
  const int S = (Nb + L - 1) / L;           // the last segment may be short
  auto bound = [&](int p) {                // first segment of part p
    if (p >= parts) return S;
    const float q = 1.f - kReplayCost;
    return (int)rintf((float)S * (1.f - __powf(q, (float)p)) / (1.f - __powf(q, (float)parts)));
  };
  const int s_att = bound(part);            // this part attends segments [s_att, s_end)
  const int s_end = bound(part + 1);
  // Lane indices, passed through an empty asm statement at the top of each
  // segment and head ("refresh") so that the addresses derived from them are
  // recomputed there instead of being kept live (and spilled) across the loop.
  int tid = threadIdx.x;
  int lane = tid & 63;
  const int wave = tid >> 6;
  int lc = lane & 15, g = lane >> 4;
  const size_t kvbase = ((size_t)b * Hkv + kvh) * N * D;

  // ---- state: M block (ab, cb) of this wave in accumulators, z in LDS
  sf32x4 macc[C::AB][C::DB];
#pragma unroll
  for (int x = 0; x < C::AB; ++x)
#pragma unroll
    for (int cb = 0; cb < C::DB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a = (wave * C::AB + x) * 16 + 4 * g + i;
        const int c = cb * 16 + lc;
        macc[x][cb][i] = M0 ? M0[(size_t)bk * D * D + (size_t)a * D + c] : 0.f;
      }
  for (int a = tid; a < D; a += 256) zs[a] = z0 ? z0[(size_t)bk * D + a] : 0.f;

  // M^T (bf16) into LDS from the accumulators: lane holds M[a0+4g..+3][c].
  auto publish_mt = [&]() {
#pragma unroll
    for (int x = 0; x < C::AB; ++x)
#pragma unroll
      for (int cb = 0; cb < C::DB; ++cb) {
        const int a = (wave * C::AB + x) * 16 + 4 * g;
        const int c = cb * 16 + lc;
        *reinterpret_cast<sbf16x4*>(Mt + c * C::MSTR + a) =
            sbf16x4{(__bf16)macc[x][cb][0], (__bf16)macc[x][cb][1], (__bf16)macc[x][cb][2], (__bf16)macc[x][cb][3]};
      }
  };

  // ---- staging of one segment's K and V: KPT keys x 8 columns per thread
  int kg = tid % C::NKG, dc = tid / C::NKG;
  sbf16x8 kst[C::KPT], vst[C::KPT];
  int Lst = L;                             // keys of the staged segment
  auto load_seg = [&](int s) {
    Lst = min(L, Nb - s * L);
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int key = min(kg * C::KPT + i, Lst - 1);
      const size_t off = kvbase + ((size_t)s * L + key) * D + dc * 8;
      kst[i] = *reinterpret_cast<const sbf16x8*>(K + off);
      vst[i] = *reinterpret_cast<const sbf16x8*>(V + off);
    }
  };
  float zp[8];
  auto store_seg = [&]() {
#pragma unroll
    for (int e = 0; e < 8; ++e) zp[e] = 0.f;
    float sk[C::KPT][8];
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const bool in = kg * C::KPT + i < Lst;
      *reinterpret_cast<sbf16x8*>(Ks + (kg * C::KPT + i) * C::KSTR + dc * 8) = kst[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = in ? elu1((float)kst[i][e]) : 0.f;
        sk[i][e] = f;
        zp[e] += f;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16* vd = Vt + (dc * 8 + e) * C::TSTR + kg * C::KPT;
      __bf16* kd = SKt + (dc * 8 + e) * C::TSTR + kg * C::KPT;
      if constexpr (C::KPT == 4) {
        // keys past the segment end carry zero V (they meet zero probability
        // and must not enter the memory update)
        const bool in0 = kg * 4 + 0 < Lst, in1 = kg * 4 + 1 < Lst, in2 = kg * 4 + 2 < Lst, in3 = kg * 4 + 3 < Lst;
        *reinterpret_cast<sbf16x4*>(vd) = sbf16x4{in0 ? vst[0][e] : (__bf16)0.f, in1 ? vst[1][e] : (__bf16)0.f,
                                                  in2 ? vst[2][e] : (__bf16)0.f, in3 ? vst[3][e] : (__bf16)0.f};
        *reinterpret_cast<sbf16x4*>(kd) = sbf16x4{(__bf16)sk[0][e], (__bf16)sk[1][e], (__bf16)sk[2][e], (__bf16)sk[3][e]};
      } else {
        const bool in0 = kg * 2 + 0 < Lst, in1 = kg * 2 + 1 < Lst;
        *reinterpret_cast<sbf16x2*>(vd) = sbf16x2{in0 ? vst[0][e] : (__bf16)0.f, in1 ? vst[1][e] : (__bf16)0.f};
        *reinterpret_cast<sbf16x2*>(kd) = sbf16x2{(__bf16)sk[0][e], (__bf16)sk[1][e]};
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) zred[kg][dc * 8 + e] = zp[e];
  };

  load_seg(0);
  store_seg();
  publish_mt();
  lds_barrier();

  int qrow = wave * 16 + lc;               // this lane's query row (the wave owns 16)
  auto refresh = [&]() { asm volatile("" : "+v"(tid), "+v"(lane), "+v"(lc), "+v"(g), "+v"(kg), "+v"(dc), "+v"(qrow)); };

  // Q^T operand of a head (lane holds query qrow, k = 32ks + 8g .. +7); the
  // group's first head is loaded one segment ahead, during the memory update
  sbf16x8 qnext[C::KS];
  auto load_q = [&](int s, int h, sbf16x8 (&qr8)[C::KS]) {
    const size_t qb = (((size_t)b * Hq + h) * N + (size_t)s * L) * D;
    const int qr = min(qrow, min(L, Nb - s * L) - 1);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qr8[ks] = *reinterpret_cast<const sbf16x8*>(Q + qb + (size_t)qr * D + ks * 32 + g * 8);
  };
  if (s_att < s_end) load_q(s_att, kvh * G, qnext);

  for (int s = 0; s < s_end; ++s) {
    refresh();
    const int Ls = min(L, Nb - s * L);     // rows and keys of this segment
    if (s + 1 < s_end) load_seg(s + 1);    // in flight while this segment computes

    for (int h = kvh * G; s >= s_att && h < (kvh + 1) * G; ++h) {
      refresh();
      const size_t qb = (((size_t)b * Hq + h) * N + (size_t)s * L) * D;
      sbf16x8 qreg[C::KS];
      if (h == kvh * G) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) qreg[ks] = qnext[ks];
      } else {
        load_q(s, h, qreg);
      }
      // S^T = K Q^T over the 4 key blocks of 16
      sf32x4 sacc[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        sacc[kb] = sf32x4{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const sbf16x8 a = *reinterpret_cast<const sbf16x8*>(Ks + (kb * 16 + lc) * C::KSTR + ks * 32 + g * 8);
          sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[ks], sacc[kb], 0, 0, 0);
        }
      }
      // exact softmax over the segment's keys: element (kb, i) is key 16kb + 4g + i
      const int lim = min(qrow, Ls - 1);
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (kb * 16 + 4 * g + i > lim) sacc[kb][i] = -INFINITY;
          mx = fmaxf(mx, sacc[kb][i]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mref = mx * sl2;
      sbf16x8 pb[2];                     // k-step t: slots 0-3 block 2t, slots 4-7 block 2t+1
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], sl2, -mref));
          const __bf16 pr = (__bf16)p;
          lsum += (float)pr;
          pb[kb >> 1][(kb & 1) * 4 + i] = pr;
        }
      lsum += __shfl_xor(lsum, 16);
      lsum += __shfl_xor(lsum, 32);
      // O^T = V^T P^T: slot 8g + q <-> key 32t + 16(q/4) + 4g + q%4
      sf32x4 oacc[C::DB];
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        oacc[db] = sf32x4{};
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const __bf16* vp = Vt + (db * 16 + lc) * C::TSTR + 32 * t + 4 * g;
          const sbf16x4 lo = *reinterpret_cast<const sbf16x4*>(vp);
          const sbf16x4 hi = *reinterpret_cast<const sbf16x4*>(vp + 16);
          const sbf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[t], oacc[db], 0, 0, 0);
        }
      }
      // retrieval from M_{s-1}: A_mem^T = M^T sigma(Q)^T, den = sigma(Q) z + eps
      sbf16x8 sq[C::KS];
      float dpart = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const __bf16 v = (__bf16)elu1((float)qreg[ks][e]);
          sq[ks][e] = v;
          dpart += (float)v * zs[ks * 32 + g * 8 + e];
        }
      dpart += __shfl_xor(dpart, 16);
      dpart += __shfl_xor(dpart, 32);
      const float den = dpart + 1e-6f;
      const float gt = sigmoid(beta[h]);
      const float wm = gt / den, wd = (1.f - gt) / lsum;
      __bf16* op = O + qb + (size_t)qrow * D;
#pragma unroll
      for (int cb = 0; cb < C::DB; ++cb) {
        sf32x4 nacc = {};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const sbf16x8 a = *reinterpret_cast<const sbf16x8*>(Mt + (cb * 16 + lc) * C::MSTR + ks * 32 + g * 8);
          nacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, sq[ks], nacc, 0, 0, 0);
        }
        if (qrow < Ls) {
          sbf16x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = (__bf16)(wm * nacc[i] + wd * oacc[cb][i]);
          *reinterpret_cast<sbf16x4*>(op + cb * 16 + 4 * g) = w;
        }
      }
      if (lse && g == 0 && qrow < Ls)
        lse[((size_t)b * Hq + h) * N + (size_t)s * L + qrow] = (mref + __log2f(lsum)) * 0.69314718055994531f;
    }
    lds_barrier();   // every read of M_{s-1}, z_{s-1} and this segment's tiles is done
    if (s + 1 < s_end && s + 1 >= s_att) load_q(s + 1, kvh * G, qnext);

    // memory update: M += sigma(K)^T V into the accumulators, z += sum sigma(K)
#pragma unroll
    for (int x = 0; x < C::AB; ++x) {
      const int ab = wave * C::AB + x;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const sbf16x8 a = *reinterpret_cast<const sbf16x8*>(SKt + (ab * 16 + lc) * C::TSTR + 32 * t + 8 * g);
#pragma unroll
        for (int cb = 0; cb < C::DB; ++cb) {
          const sbf16x8 bb = *reinterpret_cast<const sbf16x8*>(Vt + (cb * 16 + lc) * C::TSTR + 32 * t + 8 * g);
          macc[x][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb, macc[x][cb], 0, 0, 0);
        }
      }
    }
    if (tid < D) {
      float t = 0.f;
      for (int x = 0; x < C::NKG; ++x) t += zred[x][tid];
      zs[tid] += t;
    }
    lds_barrier();   // tiles and the z partials are consumed
    if (s + 1 < s_end) store_seg();
    publish_mt();
    lds_barrier();
  }
  if (part != parts - 1) return;           // the last part holds the final state

  // final state
#pragma unroll
  for (int x = 0; x < C::AB; ++x)
#pragma unroll
    for (int cb = 0; cb < C::DB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a = (wave * C::AB + x) * 16 + 4 * g + i;
        const int c = cb * 16 + lc;
        M_S[(size_t)bk * D * D + (size_t)a * D + c] = macc[x][cb][i];
      }
  for (int a = tid; a < D; a += 256) z_S[(size_t)bk * D + a] = zs[a];
}

bool fwd_short_supported(const Geometry& g) {
  return g.fmap == 0 && g.dtype == 1 && (g.D == 64 || g.D == 128) && g.L <= 64;
}

hipError_t launch_fwd_short(const Geometry& g, const void* Q, const void* K, const void* V,
                            const float* beta, const float* M0, const float* z0, void* O,
                            float* M_S, float* z_S, float* lse, hipStream_t st) {
  if (!fwd_short_supported(g)) return hipErrorInvalidValue;
  const float sl2 = 1.4426950408889634f / sqrtf((float)g.D);
  // Split each pair's segments over up to 4 workgroups (at least 2 segments
  // each on average) when the pairs alone would leave most of the 256
  // compute units idle.
  const int units = g.B * g.Hkv;
  int parts = 1;
  while (parts < 4 && parts * 4 <= g.S && units * parts * 2 <= 256) parts *= 2;
  dim3 grid(units * parts);
#define FS_ARGS static_cast<const __bf16*>(Q), static_cast<const __bf16*>(K), static_cast<const __bf16*>(V), \
                beta, M0, z0, static_cast<__bf16*>(O), M_S, z_S, lse, g.lens, g.Hq, g.Hkv, g.N, g.L, parts, sl2
  if (g.D == 128) hipLaunchKernelGGL(fwd_short_kernel<128>, grid, dim3(256), 0, st, FS_ARGS);
  else hipLaunchKernelGGL(fwd_short_kernel<64>, grid, dim3(256), 0, st, FS_ARGS);
#undef FS_ARGS
  return hipGetLastError();
}

}  // namespace infini
