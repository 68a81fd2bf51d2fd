// Fused forward for short segments (seg_len <= 64, bf16, head_dim 64 or 128).
//
// One workgroup per (batch, K/V head) walks the segments in order with the
// memory resident on chip for the whole sequence (page "Hugging Face
// Infini-Attention 재현 분석", section "Infini-Attention 메커니즘", steps
// Segmentation to State Transfer).  Its eight waves have two roles:
//   waves 4-7 own the state: M (fp32, d x d) in the accumulators of
//   v_mfma_f32_16x16x32_bf16 and z as one more product against a ones
//   operand (the sum of the same bf16 sigma(K) the update uses); per segment
//   they fold it in, M += sigma(K)^T V, z += sigma(K)^T 1, and publish the
//   bf16 M^T and z for the next segment into the other half of a
//   double-buffered LDS state;
//   waves 0-3 attend the segment, 16 query rows each, every query head of
//   the group in turn: S^T = K Q^T (all keys of the segment fit one tile, so
//   the softmax is exact, not online), O^T = V^T P^T, A_mem^T =
//   M_{s-1}^T sigma(Q)^T, den = sigma(Q) z_{s-1} + eps and the gate, one bf16
//   store.
// Both roles run at once on the same staged K and V, so a step costs the
// longer of the two, not their sum.  The update waves, whose products are
// the shorter part, also stage: after folding segment s in they write
// segment s + 1's K and V^T into the other half of double-buffered tiles
// (and its sigma(K)^T, which only they read, over segment s's) and issue the
// loads of segment s + 2, so the attention waves never stage and one barrier
// per segment suffices.  Nothing but (M, z) crosses segments and nothing but
// the final state leaves the chip.
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

constexpr float kReplayCost = 0.6f;       // replayed segment / fully processed segment

template <int D>
struct ShortCfg {
  static constexpr int BL = 64;
  static constexpr int KS = D / 32;
  static constexpr int DB = D / 16;
  static constexpr int KSTR = D + 8;
  static constexpr int TSTR = BL + 8;
  static constexpr int MSTR = D + 8;
  static constexpr int KPT = D / 32;      // keys per thread in staging (2 or 4), by the 256 update threads
  static constexpr int CH = D / 8;        // 16-byte chunks per key row
  static constexpr int AB = DB / 4;       // M row blocks per update wave
  static constexpr int KTILE = BL * KSTR;
  static constexpr int TTILE = D * TSTR;
  static constexpr int MTILE = D * MSTR;
};

template <int D>
__global__ __launch_bounds__(512)
void fwd_short_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                         const __bf16* __restrict__ V, const float* __restrict__ beta,
                         const float* __restrict__ M0, const float* __restrict__ z0,
                         __bf16* __restrict__ O, float* __restrict__ M_S, float* __restrict__ z_S,
                         float* __restrict__ lse, const int* __restrict__ lens, int Hq, int Hkv, int N, int L,
                         int parts, float sl2) {
  using C = ShortCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][C::KTILE];   // segment s in buffer s % 2
  __shared__ __attribute__((aligned(16))) __bf16 Vt[2][C::TTILE];
  __shared__ __attribute__((aligned(16))) __bf16 SKt[C::TTILE];     // read by its own writers only
  __shared__ __attribute__((aligned(16))) __bf16 Mt[2][C::MTILE];
  __shared__ __attribute__((aligned(16))) float zs[2][D];

  const int bk = blockIdx.x / parts;               // b * Hkv + kvh
  const int part = blockIdx.x % parts;
  const int b = bk / Hkv, kvh = bk % Hkv;
  const int G = Hq / Hkv;
  const int Nb = seq_len_of(lens, b, N);
  const int S = (Nb + L - 1) / L;
  auto bound = [&](int p) {
    if (p >= parts) return S;
    const float q = 1.f - kReplayCost;
    return (int)rintf((float)S * (1.f - __powf(q, (float)p)) / (1.f - __powf(q, (float)parts)));
  };
  const int s_att = bound(part);
  const int s_end = bound(part + 1);
  int tid = threadIdx.x;
  int lane = tid & 63;
  const int wave = tid >> 6;
  const bool attend_wave = wave < 4;               // uniform per wave
  const int uw = wave - 4;                         // update wave index (waves 4-7)
  int lc = lane & 15, g = lane >> 4;
  const size_t kvbase = ((size_t)b * Hkv + kvh) * N * D;

  // ---- state (update waves): M blocks and z rows in accumulators
  sf32x4 macc[C::AB][C::DB], zacc[C::AB];
  if (!attend_wave) {
#pragma unroll
    for (int x = 0; x < C::AB; ++x)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a = (uw * C::AB + x) * 16 + 4 * g + i;
        zacc[x][i] = z0 ? z0[(size_t)bk * D + a] : 0.f;
#pragma unroll
        for (int cb = 0; cb < C::DB; ++cb)
          macc[x][cb][i] = M0 ? M0[(size_t)bk * D * D + (size_t)a * D + cb * 16 + lc] : 0.f;
      }
  }
  // M^T (bf16) and z into LDS half t from the accumulators
  auto publish = [&](int t) {
#pragma unroll
    for (int x = 0; x < C::AB; ++x) {
      const int a = (uw * C::AB + x) * 16 + 4 * g;
#pragma unroll
      for (int cb = 0; cb < C::DB; ++cb)
        *reinterpret_cast<sbf16x4*>(&Mt[t][(cb * 16 + lc) * C::MSTR + a]) =
            sbf16x4{(__bf16)macc[x][cb][0], (__bf16)macc[x][cb][1], (__bf16)macc[x][cb][2], (__bf16)macc[x][cb][3]};
      if (lc == 0) *reinterpret_cast<sf32x4*>(&zs[t][a]) = zacc[x];
    }
  };

  // ---- staging of one segment's K and V by the 256 update threads; the
  // attention waves never stage.  Update wave uw stages the columns
  // (chunks dc) of K and V that hold the rows of sigma(K)^T it reads itself,
  // so sigma(K)^T needs one buffer: a wave's own LDS reads of segment s are
  // done before its writes of segment s + 1.  Thread j of the wave holds
  // chunk dc = KPT uw + j % KPT of keys kg KPT .. +KPT-1, kg = j / KPT.
  const int ut = tid - 256, uj = ut & 63;
  int dc = (ut >> 6) * C::KPT + uj % C::KPT, kg = uj / C::KPT;
  sbf16x8 kst[C::KPT], vst[C::KPT];
  int Lst = L;
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
  auto store_seg = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::KPT; ++i)
      *reinterpret_cast<sbf16x8*>(Ks[buf] + (kg * C::KPT + i) * C::KSTR + dc * 8) = kst[i];
    bool in[C::KPT];
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) in[i] = kg * C::KPT + i < Lst;
    const __bf16 zero = (__bf16)0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16* vd = Vt[buf] + (dc * 8 + e) * C::TSTR + kg * C::KPT;
      __bf16* kd = SKt + (dc * 8 + e) * C::TSTR + kg * C::KPT;
      // keys past the segment end carry zero V and zero sigma(K): they meet
      // zero probability and must not enter the memory update
      __bf16 vv[C::KPT], kk[C::KPT];
#pragma unroll
      for (int i = 0; i < C::KPT; ++i) {
        vv[i] = in[i] ? vst[i][e] : zero;
        kk[i] = in[i] ? (__bf16)elu1((float)kst[i][e]) : zero;
      }
      if constexpr (C::KPT == 2) {
        *reinterpret_cast<sbf16x2*>(vd) = sbf16x2{vv[0], vv[1]};
        *reinterpret_cast<sbf16x2*>(kd) = sbf16x2{kk[0], kk[1]};
      } else {
        *reinterpret_cast<sbf16x4*>(vd) = sbf16x4{vv[0], vv[1], vv[2], vv[3]};
        *reinterpret_cast<sbf16x4*>(kd) = sbf16x4{kk[0], kk[1], kk[2], kk[3]};
      }
    }
  };

  int qrow = wave * 16 + lc;               // attention waves: this lane's query row
  auto refresh = [&]() { asm volatile("" : "+v"(tid), "+v"(lane), "+v"(lc), "+v"(g), "+v"(kg), "+v"(dc), "+v"(qrow)); };
  sbf16x8 qnext[C::KS];
  auto load_q = [&](int s, int h, sbf16x8 (&qr8)[C::KS]) {
    const size_t qb = (((size_t)b * Hq + h) * N + (size_t)s * L) * D;
    const int qr = min(qrow, min(L, Nb - s * L) - 1);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qr8[ks] = *reinterpret_cast<const sbf16x8*>(Q + qb + (size_t)qr * D + ks * 32 + g * 8);
  };
  const sbf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                        (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};

  if (attend_wave) {
    if (s_att < s_end) load_q(s_att, kvh * G, qnext);
  } else {
    if (s_end > 0) {
      load_seg(0);
      store_seg(0);
    }
    if (s_end > 1) load_seg(1);            // in flight during segment 0
    publish(0);
  }
  lds_barrier();

  for (int s = 0; s < s_end; ++s) {
    refresh();
    const int Ls = min(L, Nb - s * L);
    const int cur = s & 1;
    const __bf16* Mts = Mt[cur];
    const float* zss = zs[cur];
    if (attend_wave) {
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
        sf32x4 sacc[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          sacc[kb] = sf32x4{};
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) {
            const sbf16x8 a = *reinterpret_cast<const sbf16x8*>(Ks[cur] + (kb * 16 + lc) * C::KSTR + ks * 32 + g * 8);
            sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[ks], sacc[kb], 0, 0, 0);
          }
        }
        const int lim = min(qrow, Ls - 1);
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (kb * 16 + 4 * g + i > lim) sacc[kb][i] = -INFINITY;
            mx = fmaxf(mx, sacc[kb][i]);
          }
        mx = quad_max(mx);
        const float mref = mx * sl2;
        sbf16x8 pb[2];
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
        lsum = quad_sum(lsum);
        sf32x4 oacc[C::DB];
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          oacc[db] = sf32x4{};
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const __bf16* vp = Vt[cur] + (db * 16 + lc) * C::TSTR + 32 * t + 4 * g;
            const sbf16x4 lo = *reinterpret_cast<const sbf16x4*>(vp);
            const sbf16x4 hi = *reinterpret_cast<const sbf16x4*>(vp + 16);
            const sbf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[t], oacc[db], 0, 0, 0);
          }
        }
        sbf16x8 sq[C::KS];
        float dpart = 0.f;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const __bf16 v = (__bf16)elu1((float)qreg[ks][e]);
            sq[ks][e] = v;
            dpart += (float)v * zss[ks * 32 + g * 8 + e];
          }
        dpart = quad_sum(dpart);
        const float den = dpart + 1e-6f;
        const float gt = sigmoid(beta[h]);
        const float wm = gt / den, wd = (1.f - gt) / lsum;
        __bf16* op = O + qb + (size_t)qrow * D;
#pragma unroll
        for (int cb = 0; cb < C::DB; ++cb) {
          sf32x4 nacc = {};
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) {
            const sbf16x8 a = *reinterpret_cast<const sbf16x8*>(Mts + (cb * 16 + lc) * C::MSTR + ks * 32 + g * 8);
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
      if (s + 1 < s_end && s + 1 >= s_att) load_q(s + 1, kvh * G, qnext);
    } else {
      // M_s = M_{s-1} + sigma(K)^T V, z_s = z_{s-1} + sigma(K)^T 1, then the
      // bf16 M_s^T and z_s for segment s + 1 into the other LDS half
#pragma unroll
      for (int x = 0; x < C::AB; ++x) {
        const int ab = uw * C::AB + x;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const sbf16x8 a = *reinterpret_cast<const sbf16x8*>(SKt + (ab * 16 + lc) * C::TSTR + 32 * t + 8 * g);
          zacc[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ones, zacc[x], 0, 0, 0);
#pragma unroll
          for (int cb = 0; cb < C::DB; ++cb) {
            const sbf16x8 bb = *reinterpret_cast<const sbf16x8*>(Vt[cur] + (cb * 16 + lc) * C::TSTR + 32 * t + 8 * g);
            macc[x][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb, macc[x][cb], 0, 0, 0);
          }
        }
      }
      publish((s + 1) & 1);
    }
    if (!attend_wave && s + 1 < s_end) {
      // segment s + 1 into the other buffers (last read in step s - 1, which
      // every wave has left), then the loads of segment s + 2
      store_seg(cur ^ 1);
      if (s + 2 < s_end) load_seg(s + 2);
    }
    lds_barrier();   // segment s's tiles and M_{s-1}^T are consumed; M_s^T and segment s + 1 are in place
  }
  if (part != parts - 1 || attend_wave) return;    // the last part's update waves hold the final state
#pragma unroll
  for (int x = 0; x < C::AB; ++x)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int a = (uw * C::AB + x) * 16 + 4 * g + i;
#pragma unroll
      for (int cb = 0; cb < C::DB; ++cb) M_S[(size_t)bk * D * D + (size_t)a * D + cb * 16 + lc] = macc[x][cb][i];
      if (lc == 0) z_S[(size_t)bk * D + a] = zacc[x][i];
    }
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
  if (g.D == 128) hipLaunchKernelGGL(fwd_short_kernel<128>, grid, dim3(512), 0, st, FS_ARGS);
  else hipLaunchKernelGGL(fwd_short_kernel<64>, grid, dim3(512), 0, st, FS_ARGS);
#undef FS_ARGS
  return hipGetLastError();
}

}  // namespace infini
