// Matrix-core forward for the second-order Taylor feature map (bf16, head
// dim 64 or 128).
//
// Page "Based" (cartesia.ai), section "고정 크기 순환 상태를 사용하는 방법도
// 중요합니다": phi is chosen so that phi(q) . phi(k) = 1 + q.k + (q.k)^2 / 2,
// and the key dimension grows to about d^2; section "I/O와 데이터 흐름을
// 고려한 구현" notes that the resulting O(N d'^2 d) state makes a plain
// implementation slow.  This file never forms the per-segment states at
// all.  The memory before segment s is M_0 plus the sum over the earlier
// tokens j of phi(k_j)^T v_j (and z_0 plus the sum of phi(k_j)), so the
// retrieval of page "Hugging Face Infini-Attention 재현 분석", section
// "Infini-Attention 메커니즘" (Memory Retrieval) is, for a query q of
// segment s,
//   A_mem = (phi(q) M_0 + sum_j kappa(q.k_j) v_j)
//           / (phi(q) z_0 + sum_j kappa(q.k_j) + eps),
//   kappa(t) = phi(q) . phi(k) = 1 + t + t^2 / 2,
// over the keys j before the segment's first token: an attention over the
// earlier segments with polynomial weights instead of exponentials, the
// same order of work as the local attention itself, plus, with a starting
// state, one product of phi(q) with it per query (taylor_m0_kernel).
//
// One launch, taylor_fwd_kernel, with two kinds of workgroup side by side:
//   attention items      one workgroup of 4 waves per 64 query rows of a
//                        (batch, query head, segment): key tiles of 64 staged
//                        in LDS (K row-major, V^T), S^T = K Q^T and
//                        O^T = V^T P^T on v_mfma_f32_16x16x32_bf16; the tiles
//                        before the segment take the weights kappa(S), the
//                        segment's own tiles the causal online softmax of
//                        S / sqrt d; then the gate, one bf16 store.
//   state workgroups     the state after the call, M_S = sum_j phi(k_j)^T v_j
//                        and z_S = sum_j phi(k_j) (D' = 1 + d + d^2 rows),
//                        which the call returns: one wave per task and 64
//                        value columns, a task being the quadratic rows
//                        k_a k_b / sqrt 2 of a and of d-1-a from the 16-row
//                        block of each upwards (the rows below are written
//                        as their mirrors), or the constant and linear rows;
//                        the operand k_a * k_b is formed in registers from
//                        the staged K^T, z as one more product against a
//                        ones operand.
//
// 16x16x32 bf16 operand layout (gfx950): A lane l holds row l%16, k = 8(l/16)..+7;
// B lane l holds column l%16, same k; C/D lane l holds column l%16,
// rows 4(l/16) + i, i = 0..3.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace infini {

namespace {

typedef __bf16 tbf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 tbf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 tbf16x2 __attribute__((ext_vector_type(2)));
typedef float tf32x4 __attribute__((ext_vector_type(4)));

constexpr float kTRsqrt2 = 0.70710678118654752f;

template <int D>
struct TaCfg {
  static constexpr int BQ = 64;          // query rows per workgroup (4 waves x 16)
  static constexpr int BK = 64;          // keys per staged tile
  static constexpr int KS = D / 32;      // k-steps of the score products
  static constexpr int DB = D / 16;      // 16-row blocks of the value dim
  static constexpr int KSTR = D + 8;     // staged K row stride (bf16)
  static constexpr int TSTR = BK + 8;    // staged V^T / K^T row stride
  static constexpr int KPT = D / 32;     // keys per thread in staging (256 threads)
  static constexpr int CH = D / 8;       // 16-byte chunks per key row
  static constexpr int KTILE = BK * KSTR;
  static constexpr int TTILE = D * TSTR;
};

}  // namespace

// Attention work item w (longest first: the latest segments carry the most
// earlier keys) -> (segment, batch, query head, query tile).
template <int D>
__device__ __forceinline__ void taylor_attn_item(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const float* __restrict__ beta, __bf16* __restrict__ O, float* __restrict__ lse,
    const int* __restrict__ lens, const float* __restrict__ num0, const float* __restrict__ den0, int B, int Hq,
    int Hkv, int N, int L, int S, int T, float sl2, int w, __bf16 (*Ks)[TaCfg<D>::KTILE],
    __bf16 (*Vt)[TaCfg<D>::TTILE]) {
  using C = TaCfg<D>;
  const int per_s = B * Hq * T;
  const int s = S - 1 - w / per_s;
  int r = w % per_s;
  const int t = r % T;
  r /= T;
  const int h = r % Hq, b = r / Hq;
  const int G = Hq / Hkv, kvh = h / G;
  const int Nb = seq_len_of(lens, b, N);
  const int seg0 = s * L;
  if (seg0 >= Nb) return;                          // uniform: the whole workgroup leaves
  const int Ls = min(L, Nb - seg0);
  const int q0 = t * C::BQ;                        // first query row of the tile in the segment
  if (q0 >= Ls) return;
  const int qn = min(C::BQ, Ls - q0);
  const int np = (seg0 + C::BK - 1) / C::BK;       // tiles of earlier keys
  const int nl = (min(Ls, q0 + qn) + C::BK - 1) / C::BK;   // causal tiles of the segment
  const int ntiles = np + nl;

  int tid = threadIdx.x;
  int lane = tid & 63;
  const int wave = tid >> 6;
  int lc = lane & 15, g = lane >> 4;
  const size_t kvbase = ((size_t)b * Hkv + kvh) * N * D;

  // staging: thread holds 8 columns (chunk dc) of keys kg*KPT .. +KPT-1 of K
  // and V; a wave's load covers whole key rows
  int dc = tid % C::CH, kg = tid / C::CH;
  tbf16x8 kst[C::KPT], vst[C::KPT];
  auto tile_key0 = [&](int j) { return j < np ? j * C::BK : seg0 + (j - np) * C::BK; };
  auto tile_end = [&](int j) { return j < np ? seg0 : seg0 + Ls; };
  auto load_tile = [&](int j) {
    const int k0 = tile_key0(j), kl = tile_end(j) - 1;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int key = min(k0 + kg * C::KPT + i, kl);
      const size_t off = kvbase + (size_t)key * D + dc * 8;
      kst[i] = *reinterpret_cast<const tbf16x8*>(K + off);
      vst[i] = *reinterpret_cast<const tbf16x8*>(V + off);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::KPT; ++i)
      *reinterpret_cast<tbf16x8*>(Ks[buf] + (kg * C::KPT + i) * C::KSTR + dc * 8) = kst[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16* vd = Vt[buf] + (dc * 8 + e) * C::TSTR + kg * C::KPT;
      if constexpr (C::KPT == 2) {
        *reinterpret_cast<tbf16x2*>(vd) = tbf16x2{vst[0][e], vst[1][e]};
      } else {
        *reinterpret_cast<tbf16x4*>(vd) = tbf16x4{vst[0][e], vst[1][e], vst[2][e], vst[3][e]};
      }
    }
  };

  int qrow = q0 + wave * 16 + lc;                  // this lane's query row in the segment
  auto refresh = [&]() { asm volatile("" : "+v"(tid), "+v"(lane), "+v"(lc), "+v"(g), "+v"(kg), "+v"(dc), "+v"(qrow)); };
  const size_t qb = (((size_t)b * Hq + h) * N + seg0) * D;
  tbf16x8 qreg[C::KS];
  {
    const int qr = min(qrow, Ls - 1);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qreg[ks] = *reinterpret_cast<const tbf16x8*>(Q + qb + (size_t)qr * D + ks * 32 + g * 8);
  }

  tf32x4 omem[C::DB], odot[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) omem[db] = odot[db] = tf32x4{};
  float den = 0.f, lsum = 0.f, mref = -INFINITY;   // lane partials; mref in base-2 units

  load_tile(0);
  store_tile(0);
  lds_barrier();
  for (int j = 0; j < ntiles; ++j) {
    refresh();
    const int buf = j & 1;
    if (j + 1 < ntiles) load_tile(j + 1);          // in flight while this tile computes
    const __bf16* Kb = Ks[buf];
    const __bf16* Vb = Vt[buf];
    tf32x4 sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[kb] = tf32x4{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const tbf16x8 a = *reinterpret_cast<const tbf16x8*>(Kb + (kb * 16 + lc) * C::KSTR + ks * 32 + g * 8);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[ks], sacc[kb], 0, 0, 0);
      }
    }
    const int k0 = tile_key0(j);
    tbf16x8 pb[2];
    if (j < np) {
      // earlier segments: weight kappa(q.k), keys at or past the segment start excluded
      const int lim = seg0 - k0;                   // keys of the tile below it
      if (lim >= C::BK) {                          // uniform: a whole tile of earlier keys
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = sacc[kb][i];
            const __bf16 wr = (__bf16)fmaf(x, fmaf(x, 0.5f, 1.f), 1.f);
            den += (float)wr;
            pb[kb >> 1][(kb & 1) * 4 + i] = wr;
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = sacc[kb][i];
            const float w = kb * 16 + 4 * g + i < lim ? fmaf(x, fmaf(x, 0.5f, 1.f), 1.f) : 0.f;
            const __bf16 wr = (__bf16)w;
            den += (float)wr;
            pb[kb >> 1][(kb & 1) * 4 + i] = wr;
          }
      }
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const __bf16* vp = Vb + (db * 16 + lc) * C::TSTR + 32 * tt + 4 * g;
          const tbf16x4 lo = *reinterpret_cast<const tbf16x4*>(vp);
          const tbf16x4 hi = *reinterpret_cast<const tbf16x4*>(vp + 16);
          const tbf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          omem[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[tt], omem[db], 0, 0, 0);
        }
    } else {
      // the segment itself: causal online softmax of S / sqrt d
      const int lim = min(qrow, Ls - 1) - (k0 - seg0);
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (kb * 16 + 4 * g + i > lim) sacc[kb][i] = -INFINITY;
          mx = fmaxf(mx, sacc[kb][i]);
        }
      mx = quad_max(mx);
      const float mnew = fmaxf(mref, mx * sl2);    // finite from the segment's first tile on
      const float alpha = __builtin_amdgcn_exp2f(mref - mnew);
      mref = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) odot[db] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const __bf16 pr = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[kb][i], sl2, -mnew));
          lsum += (float)pr;
          pb[kb >> 1][(kb & 1) * 4 + i] = pr;
        }
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const __bf16* vp = Vb + (db * 16 + lc) * C::TSTR + 32 * tt + 4 * g;
          const tbf16x4 lo = *reinterpret_cast<const tbf16x4*>(vp);
          const tbf16x4 hi = *reinterpret_cast<const tbf16x4*>(vp + 16);
          const tbf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          odot[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[tt], odot[db], 0, 0, 0);
        }
    }
    // the other buffer was last read in step j - 1, which every wave has left
    if (j + 1 < ntiles) store_tile(buf ^ 1);
    lds_barrier();
  }

  den = quad_sum(den);
  lsum = quad_sum(lsum);
  if (num0 && qrow < Ls) {                         // the starting state's part of the retrieval
    const size_t r = ((size_t)b * Hq + h) * N + seg0 + qrow;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const float4 n4 = *reinterpret_cast<const float4*>(num0 + r * D + db * 16 + 4 * g);
      omem[db] += tf32x4{n4.x, n4.y, n4.z, n4.w};
    }
    den += den0[r];
  }
  const float gt = sigmoid(beta[h]);
  const float wm = gt / (den + 1e-6f), wd = (1.f - gt) / lsum;
  if (qrow < Ls) {
    __bf16* op = O + qb + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      tbf16x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (__bf16)(wm * omem[db][i] + wd * odot[db][i]);
      *reinterpret_cast<tbf16x4*>(op + db * 16 + 4 * g) = w;
    }
    if (lse && g == 0) lse[((size_t)b * Hq + h) * N + seg0 + qrow] = (mref + __log2f(lsum)) * 0.69314718055994531f;
  }
}

// The state after the call, row order of phi: row 0 the constant 1, rows
// 1..D the linear features k_b, rows 1 + D + a D + b the quadratic features
// k_a k_b / sqrt 2.  Quadratic rows (a, b) and (b, a) hold the same sums, so
// only the 16-row blocks with b at or above the 16-block of a are formed
// and the rest are written as their mirror.
//
// One wave per task and 64 value columns, 4 waves per workgroup, every key of
// the sequence in staged tiles of 64 (K^T and V^T in LDS; K^T row D holds 1
// for keys in range, 0 past the end).  Task p < D/2 of a (batch, K/V head)
// owns the quadratic rows of a0 = p (blocks a0/16 .. DB-1) and of
// a1 = D-1-p (blocks a1/16 .. DB-1): DB + 1 blocks of 16 rows.  Task D/2
// owns the linear rows (DB blocks) and the constant row (one block whose
// operand rows are all the ones row): DB + 1 blocks as well, so every wave
// does the same work.  The operand k_a k_b of a block is formed in registers
// from the staged K^T with v_dot2_f32_bf16 against (k_a, 0) and (0, k_a)
// pairs (each result is one exact product, rounded once to bf16); z is one
// more product against a ones operand.
template <int D>
struct TsCfg {
  static constexpr int DB = D / 16;
  static constexpr int NX = DB + 1;                // 16-row blocks per task
  static constexpr int CB = 4;                     // 16-column blocks per task (64 columns)
  static constexpr int NCH = D / 64;               // 64-column halves of the value dim
  static constexpr int NTASK = (D / 2 + 1) * NCH;  // tasks per (batch, K/V head)
  static constexpr int TSTR = 72;                  // staged K^T / V^T row stride (bf16)
  static constexpr int KPT = D / 32;               // keys per thread in staging (256 threads)
  static constexpr int CH = D / 8;                 // 16-byte chunks per key row
  static constexpr bool PREFETCH = D == 64;
};

// a.x b.x + a.y b.y in fp32 (v_dot2_f32_bf16) with a zero addend: with one
// of b's halves zero it is one exact product.
__device__ __forceinline__ float dot2_exact(tbf16x2 a, tbf16x2 b) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, 0.f, false);
}

// One 64-key tile of a task.  P: 16-block index of a0 (0 .. DB/2 - 1), or -1
// for the linear task.
template <int D, int P>
__device__ __forceinline__ void state_tile(const __bf16* __restrict__ KTb, const __bf16* __restrict__ VTb, int a0,
                                           int a1, int c0, bool do_z, int lc, int g,
                                           tf32x4 (&macc)[TsCfg<D>::NX][TsCfg<D>::CB],
                                           tf32x4 (&zacc)[TsCfg<D>::NX]) {
  using C = TsCfg<D>;
  constexpr int NA = P < 0 ? C::DB : C::DB - P;    // blocks of a0 (or the linear blocks)
  constexpr int B1 = C::DB - 1 - P;                // 16-block of a1
  const tbf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                        (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
#pragma nounroll
  for (int tt = 0; tt < 2; ++tt) {
    const int kc = 32 * tt + 8 * g;
    tbf16x8 vb[C::CB];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
      vb[cb] = *reinterpret_cast<const tbf16x8*>(VTb + (c0 + cb * 16 + lc) * C::TSTR + kc);
    // (k_a, 0) and (0, k_a) pairs of the multiplier rows
    tbf16x2 m0[8], m1[8];
    if constexpr (P >= 0) {
      const tbf16x8 r0 = *reinterpret_cast<const tbf16x8*>(KTb + a0 * C::TSTR + kc);
      const tbf16x8 r1 = *reinterpret_cast<const tbf16x8*>(KTb + a1 * C::TSTR + kc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const __bf16 z = (__bf16)0.f;
        m0[2 * e] = tbf16x2{r0[2 * e], z};
        m0[2 * e + 1] = tbf16x2{z, r0[2 * e + 1]};
        m1[2 * e] = tbf16x2{r1[2 * e], z};
        m1[2 * e + 1] = tbf16x2{z, r1[2 * e + 1]};
      }
    }
    auto krow_of = [&](int x) {
      if constexpr (P < 0) return x < C::DB ? x * 16 + lc : D;
      else return (x < NA ? (P + x) * 16 : (B1 + x - NA) * 16) + lc;
    };
    if constexpr (P < 0) {
#pragma unroll
      for (int x = 0; x < C::NX; ++x) {
        // times the ones row: the linear features themselves
        const tbf16x8 op = *reinterpret_cast<const tbf16x8*>(KTb + krow_of(x) * C::TSTR + kc);
        if (do_z) zacc[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op, ones, zacc[x], 0, 0, 0);
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
          macc[x][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op, vb[cb], macc[x][cb], 0, 0, 0);
      }
    } else {
      tbf16x8 kr[C::NX];
#pragma unroll
      for (int x = 0; x < C::NX; ++x) kr[x] = *reinterpret_cast<const tbf16x8*>(KTb + krow_of(x) * C::TSTR + kc);
      // products k_a k_b of pair e of block x
      auto form = [&](int x, int e) {
        const tbf16x2 kp = {kr[x][2 * e], kr[x][2 * e + 1]};
        const float lo = dot2_exact(kp, x < NA ? m0[2 * e] : m1[2 * e]);
        const float hi = dot2_exact(kp, x < NA ? m0[2 * e + 1] : m1[2 * e + 1]);
        return tbf16x2{(__bf16)lo, (__bf16)hi};
      };
      tbf16x8 op;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const tbf16x2 w = form(0, e);
        op[2 * e] = w[0];
        op[2 * e + 1] = w[1];
      }
      // the matrix products of block x, with block x + 1's operand formed
      // beside them
#pragma unroll
      for (int x = 0; x < C::NX; ++x) {
        tbf16x8 nop = op;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
          macc[x][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op, vb[cb], macc[x][cb], 0, 0, 0);
          if (x + 1 < C::NX) {
            const tbf16x2 w = form(x + 1, cb);
            nop[2 * cb] = w[0];
            nop[2 * cb + 1] = w[1];
          }
        }
        if (do_z) zacc[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op, ones, zacc[x], 0, 0, 0);
        op = nop;
      }
    }
  }
}

// Writes a task's blocks (and their mirrors) into M_S / z_S of one (batch, K/V head).
template <int D, int P>
// M0b / z0b: the starting state of the same (batch, K/V head), added to
// every entry, or NULL.
__device__ __forceinline__ void state_store(float* __restrict__ Mb, float* __restrict__ zb,
                                            const float* __restrict__ M0b, const float* __restrict__ z0b, int a0,
                                            int a1, int c0, int Nb, int lc, int g,
                                            const tf32x4 (&macc)[TsCfg<D>::NX][TsCfg<D>::CB],
                                            const tf32x4 (&zacc)[TsCfg<D>::NX]) {
  using C = TsCfg<D>;
  auto m0 = [&](size_t i) { return M0b ? M0b[i] : 0.f; };
  auto z0 = [&](size_t i) { return z0b ? z0b[i] : 0.f; };
  constexpr int NA = P < 0 ? C::DB : C::DB - P;
  constexpr int B1 = C::DB - 1 - P;
  const bool zl = c0 == 0 && lc == 0;
#pragma unroll
  for (int x = 0; x < C::NX; ++x) {
    if constexpr (P < 0) {
      if (x < C::DB) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 1 + x * 16 + 4 * g + i;
#pragma unroll
          for (int cb = 0; cb < C::CB; ++cb) {
            const size_t o = (size_t)row * D + c0 + cb * 16 + lc;
            Mb[o] = m0(o) + macc[x][cb][i];
          }
          if (zl) zb[row] = z0(row) + zacc[x][i];
        }
      } else if (g == 0) {                         // constant row: every row of the block holds it
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) Mb[c0 + cb * 16 + lc] = m0(c0 + cb * 16 + lc) + macc[x][cb][0];
        if (zl) zb[0] = z0(0) + (float)Nb;
      }
    } else {
      const int a = x < NA ? a0 : a1;
      const int bb = x < NA ? P + x : B1 + x - NA;
      const bool mirror = x < NA ? x > 0 : x > NA;  // block above the diagonal block of a
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = bb * 16 + 4 * g + i;
        const size_t r1 = 1 + D + (size_t)a * D + b, r2 = 1 + D + (size_t)b * D + a;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
          const float v = kTRsqrt2 * macc[x][cb][i];
          const size_t o1 = r1 * D + c0 + cb * 16 + lc, o2 = r2 * D + c0 + cb * 16 + lc;
          Mb[o1] = m0(o1) + v;
          if (mirror) Mb[o2] = m0(o2) + v;
        }
        if (zl) {
          const float v = kTRsqrt2 * zacc[x][i];
          zb[r1] = z0(r1) + v;
          if (mirror) zb[r2] = z0(r2) + v;
        }
      }
    }
  }
}

// The whole pass of one workgroup whose tasks all have variant P (so every
// wave of it runs the same code and the same barriers).  task: this wave's
// task (pair index and column half), or -1 for an idle wave.
template <int D, int P>
__device__ __forceinline__ void state_pass(const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                                           float* __restrict__ Mb, float* __restrict__ zb,
                                           const float* __restrict__ M0b, const float* __restrict__ z0b, int Nb,
                                           size_t kvbase, int task, __bf16 (*KT)[(D + 1) * TsCfg<D>::TSTR],
                                           __bf16 (*VT)[D * TsCfg<D>::TSTR]) {
  using C = TsCfg<D>;

  int tid = threadIdx.x;
  int lane = tid & 63;
  int lc = lane & 15, g = lane >> 4;
  const bool active = task >= 0;                    // uniform per wave
  const int pt = task / C::NCH;
  const int c0 = (task % C::NCH) * 64;
  const bool do_z = c0 == 0;
  const int a0 = P < 0 ? 0 : pt, a1 = P < 0 ? 0 : D - 1 - pt;

  int dc = tid % C::CH, kg = tid / C::CH;           // chunk dc of keys kg*KPT ..: whole rows per wave
  tbf16x8 kst[C::KPT], vst[C::KPT];
  int kvalid = 0;
  auto load_tile = [&](int j) {
    const int k0 = j * 64;
    kvalid = Nb - k0;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int key = min(k0 + kg * C::KPT + i, Nb - 1);
      const size_t off = kvbase + (size_t)key * D + dc * 8;
      kst[i] = *reinterpret_cast<const tbf16x8*>(K + off);
      vst[i] = *reinterpret_cast<const tbf16x8*>(V + off);
    }
  };
  // keys past the sequence end carry zero K^T and V^T columns and a 0 in the
  // ones row, so they add nothing to any sum
  auto store_tile = [&](int buf) {
    bool in[C::KPT];
    const bool full = kvalid >= 64;                 // uniform: no key of the tile past the end
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) in[i] = full || kg * C::KPT + i < kvalid;
    const __bf16 zero = (__bf16)0.f, one = (__bf16)1.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16* vd = VT[buf] + (dc * 8 + e) * C::TSTR + kg * C::KPT;
      __bf16* kd = KT[buf] + (dc * 8 + e) * C::TSTR + kg * C::KPT;
      if constexpr (C::KPT == 2) {
        *reinterpret_cast<tbf16x2*>(vd) = tbf16x2{in[0] ? vst[0][e] : zero, in[1] ? vst[1][e] : zero};
        *reinterpret_cast<tbf16x2*>(kd) = tbf16x2{in[0] ? kst[0][e] : zero, in[1] ? kst[1][e] : zero};
      } else {
        *reinterpret_cast<tbf16x4*>(vd) = tbf16x4{in[0] ? vst[0][e] : zero, in[1] ? vst[1][e] : zero,
                                                  in[2] ? vst[2][e] : zero, in[3] ? vst[3][e] : zero};
        *reinterpret_cast<tbf16x4*>(kd) = tbf16x4{in[0] ? kst[0][e] : zero, in[1] ? kst[1][e] : zero,
                                                  in[2] ? kst[2][e] : zero, in[3] ? kst[3][e] : zero};
      }
    }
    if (dc == 0) {
      __bf16* od = KT[buf] + D * C::TSTR + kg * C::KPT;
      if constexpr (C::KPT == 2) {
        *reinterpret_cast<tbf16x2*>(od) = tbf16x2{in[0] ? one : zero, in[1] ? one : zero};
      } else {
        *reinterpret_cast<tbf16x4*>(od) = tbf16x4{in[0] ? one : zero, in[1] ? one : zero, in[2] ? one : zero,
                                                  in[3] ? one : zero};
      }
    }
  };
  auto refresh = [&]() { asm volatile("" : "+v"(tid), "+v"(lane), "+v"(lc), "+v"(g), "+v"(kg), "+v"(dc)); };

  tf32x4 macc[C::NX][C::CB], zacc[C::NX];
#pragma unroll
  for (int x = 0; x < C::NX; ++x) {
    zacc[x] = tf32x4{};
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) macc[x][cb] = tf32x4{};
  }

  const int ntiles = (Nb + 63) / 64;
  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  lds_barrier();
  for (int j = 0; j < ntiles; ++j) {
    refresh();
    const int buf = j & 1;
    // head_dim 64 has the registers to keep the next tile's loads in flight
    // during this tile's products; head_dim 128 issues them afterwards
    if (C::PREFETCH && j + 1 < ntiles) load_tile(j + 1);
    if (active) state_tile<D, P>(KT[buf], VT[buf], a0, a1, c0, do_z, lc, g, macc, zacc);
    // the other buffer was last read in step j - 1, which every wave has left
    if (j + 1 < ntiles) {
      if (!C::PREFETCH) load_tile(j + 1);
      store_tile(buf ^ 1);
    }
    lds_barrier();
  }
  if (active) state_store<D, P>(Mb, zb, M0b, z0b, a0, a1, c0, Nb, lc, g, macc, zacc);
}

// State workgroup of launch index wid.  Workgroups of a (batch, K/V head):
// for each 16-block P of the pair index, 4 * NCH workgroups of 4 pair tasks
// (16 pairs x NCH column halves), then one workgroup for the linear task's
// NCH column halves.
template <int D>
__device__ __forceinline__ void taylor_state_item(
    const __bf16* __restrict__ K, const __bf16* __restrict__ V, const float* __restrict__ M0,
    const float* __restrict__ z0, float* __restrict__ M_S, float* __restrict__ z_S, const int* __restrict__ lens,
    int Hkv, int N, int wg_per_bk, int items, int per_xcd, int wid, __bf16 (*KT)[(D + 1) * TsCfg<D>::TSTR],
    __bf16 (*VT)[D * TsCfg<D>::TSTR]) {
  using C = TsCfg<D>;
  constexpr size_t DF = 1 + (size_t)D + (size_t)D * D;
  constexpr int WP = 4 * C::NCH;                    // workgroups per 16-block of pairs
  // workgroups go to the 8 XCDs in turn (launch index % 8); item numbers are
  // contiguous per XCD, so the workgroups of one (batch, K/V head), which all
  // read its K and V, share one XCD's L2
  const int item = (wid % 8) * per_xcd + wid / 8;
  if (item >= items) return;                        // uniform
  const int bk = item / wg_per_bk;
  const int wg = item % wg_per_bk;
  const int Nb = seq_len_of(lens, bk / Hkv, N);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  float* Mb = M_S + (size_t)bk * DF * D;
  float* zb = z_S + (size_t)bk * DF;
  const float* M0b = M0 ? M0 + (size_t)bk * DF * D : nullptr;
  const float* z0b = z0 ? z0 + (size_t)bk * DF : nullptr;
  const size_t kvbase = (size_t)bk * N * D;
  const int P = wg / WP;                            // D/32 for the linear workgroup
  if (P >= D / 32) {
    state_pass<D, -1>(K, V, Mb, zb, M0b, z0b, Nb, kvbase, wave < C::NCH ? (D / 2) * C::NCH + wave : -1, KT, VT);
    return;
  }
  const int task = (P * 16) * C::NCH + (wg % WP) * 4 + wave;   // pair P*16 + l / NCH, half l % NCH
  switch (P) {
    case 0: state_pass<D, 0>(K, V, Mb, zb, M0b, z0b, Nb, kvbase, task, KT, VT); break;
    case 1: state_pass<D, 1>(K, V, Mb, zb, M0b, z0b, Nb, kvbase, task, KT, VT); break;
    case 2: if constexpr (D >= 128) state_pass<D, 2>(K, V, Mb, zb, M0b, z0b, Nb, kvbase, task, KT, VT); break;
    case 3: if constexpr (D >= 128) state_pass<D, 3>(K, V, Mb, zb, M0b, z0b, Nb, kvbase, task, KT, VT); break;
    default: break;
  }
}

// The starting state's part of the retrieval, phi(q) M_0 and phi(q) z_0, of
// every query row, into num0 [B][Hq][N][D] and den0 [B][Hq][N] (fp32) for
// the attention items to add.  One workgroup of 4 waves per 256 query rows
// of a (batch, query head), each wave 4 blocks of 16 rows.  The state is
// walked one feature group at a time, each group staged in LDS as bf16
// [value column][feature]: the linear rows 1..D, then quadratic group a
// (rows 1 + D + a D + b, scaled by 1/sqrt 2 before rounding).  The operand
// phi(q) of a group is formed in registers: q_b itself, or q_a q_b by
// v_dot2_f32_bf16 against (q_a, 0) / (0, q_a) pairs; the den part is one
// more product whose A rows all hold the group's z entries.  The constant
// row is added in fp32.
template <int D>
struct TmCfg {
  static constexpr int QB = 4;                     // 16-row query blocks per wave
  static constexpr int ROWS = 64 * QB;             // query rows per workgroup
  static constexpr int DB = D / 16, KS = D / 32;
  static constexpr int MSTR = D + 8;               // staged group: rows = value columns, bf16
  static constexpr int QSTR = D + 8;               // staged query rows
};

template <int D>
__global__ __launch_bounds__(256) void taylor_m0_kernel(
    const __bf16* __restrict__ Q, const float* __restrict__ M0, const float* __restrict__ z0,
    float* __restrict__ num0, float* __restrict__ den0, const int* __restrict__ lens, int Hq, int Hkv, int N,
    int tiles) {
  using C = TmCfg<D>;
  constexpr size_t DF = 1 + (size_t)D + (size_t)D * D;
  __shared__ __attribute__((aligned(16))) __bf16 Mt[D * C::MSTR];
  __shared__ __attribute__((aligned(16))) __bf16 zt[D];
  __shared__ __attribute__((aligned(16))) __bf16 Qs[C::ROWS * C::QSTR];
  const int bh = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  const int b = bh / Hq, h = bh % Hq;
  const int bk = b * Hkv + h / (Hq / Hkv);
  const int Nb = seq_len_of(lens, b, N);
  const int r0 = tile * C::ROWS;
  if (r0 >= Nb) return;                            // uniform
  const float* M0b = M0 + (size_t)bk * DF * D;
  const float* z0b = z0 + (size_t)bk * DF;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lc = lane & 15, g = lane >> 4;
  const size_t qbase = (size_t)bh * N * D;
  // the tile's query rows (rows past the sequence repeat its last row)
  for (int idx = tid; idx < C::ROWS * (D / 8); idx += 256) {
    const int r = idx / (D / 8), c8 = idx % (D / 8);
    const int q = min(r0 + r, Nb - 1);
    *reinterpret_cast<tbf16x8*>(Qs + r * C::QSTR + c8 * 8) =
        *reinterpret_cast<const tbf16x8*>(Q + qbase + (size_t)q * D + c8 * 8);
  }
  tf32x4 acc[C::QB][C::DB], zac[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    zac[qb] = tf32x4{};
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[qb][db] = tf32x4{};
  }
  const __bf16 zero = (__bf16)0.f;
  for (int grp = 0; grp <= D; ++grp) {             // 0: linear rows; 1 + a: quadratic group a
    const size_t frow = grp == 0 ? 1 : 1 + D + (size_t)(grp - 1) * D;
    const float sc = grp == 0 ? 1.f : kTRsqrt2;
    lds_barrier();                                  // the previous group's reads are done
    for (int idx = tid; idx < (D / 4) * (D / 4); idx += 256) {
      const int f4 = idx / (D / 4), c4 = idx % (D / 4);
      float4 rw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) rw[j] = *reinterpret_cast<const float4*>(M0b + (frow + f4 * 4 + j) * D + c4 * 4);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const float v0 = cc == 0 ? rw[0].x : cc == 1 ? rw[0].y : cc == 2 ? rw[0].z : rw[0].w;
        const float v1 = cc == 0 ? rw[1].x : cc == 1 ? rw[1].y : cc == 2 ? rw[1].z : rw[1].w;
        const float v2 = cc == 0 ? rw[2].x : cc == 1 ? rw[2].y : cc == 2 ? rw[2].z : rw[2].w;
        const float v3 = cc == 0 ? rw[3].x : cc == 1 ? rw[3].y : cc == 2 ? rw[3].z : rw[3].w;
        *reinterpret_cast<tbf16x4*>(Mt + (c4 * 4 + cc) * C::MSTR + f4 * 4) =
            tbf16x4{(__bf16)(sc * v0), (__bf16)(sc * v1), (__bf16)(sc * v2), (__bf16)(sc * v3)};
      }
    }
    if (tid < D) zt[tid] = (__bf16)(sc * z0b[frow + tid]);
    lds_barrier();
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      const int qr = wave * 64 + qb * 16 + lc;
      const __bf16 qa = grp == 0 ? zero : Qs[qr * C::QSTR + grp - 1];
      const tbf16x2 mlo = {qa, zero}, mhi = {zero, qa};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const tbf16x8 qv = *reinterpret_cast<const tbf16x8*>(Qs + qr * C::QSTR + ks * 32 + 8 * g);
        tbf16x8 op = qv;
        if (grp > 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const tbf16x2 kp = {qv[2 * e], qv[2 * e + 1]};
            op[2 * e] = (__bf16)dot2_exact(kp, mlo);
            op[2 * e + 1] = (__bf16)dot2_exact(kp, mhi);
          }
        }
        const tbf16x8 za = *reinterpret_cast<const tbf16x8*>(zt + ks * 32 + 8 * g);
        zac[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(za, op, zac[qb], 0, 0, 0);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const tbf16x8 a = *reinterpret_cast<const tbf16x8*>(Mt + (db * 16 + lc) * C::MSTR + ks * 32 + 8 * g);
          acc[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, op, acc[qb][db], 0, 0, 0);
        }
      }
    }
  }
  // the constant row, then the stores
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int q = r0 + wave * 64 + qb * 16 + lc;
    if (q >= Nb) continue;
    const size_t r = (size_t)bh * N + q;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const float4 m = *reinterpret_cast<const float4*>(M0b + db * 16 + 4 * g);
      *reinterpret_cast<float4*>(num0 + r * D + db * 16 + 4 * g) =
          float4{acc[qb][db][0] + m.x, acc[qb][db][1] + m.y, acc[qb][db][2] + m.z, acc[qb][db][3] + m.w};
    }
    if (g == 0) den0[r] = zac[qb][0] + z0b[0];
  }
}

// One launch for both: the state workgroups first (8 * per_xcd of them,
// the longest), then the attention items; the two kinds run side by side.
template <int D>
struct TfLds {
  static constexpr size_t ATT = 2 * (TaCfg<D>::KTILE + TaCfg<D>::TTILE) * sizeof(__bf16);
  static constexpr size_t ST = 2 * ((D + 1) * TsCfg<D>::TSTR + D * TsCfg<D>::TSTR) * sizeof(__bf16);
  static constexpr size_t BYTES = ATT > ST ? ATT : ST;
};

template <int D>
__global__ __launch_bounds__(256) void taylor_fwd_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const float* __restrict__ beta, const float* __restrict__ M0, const float* __restrict__ z0,
    const float* __restrict__ num0, const float* __restrict__ den0, __bf16* __restrict__ O, float* __restrict__ lse,
    float* __restrict__ M_S, float* __restrict__ z_S, const int* __restrict__ lens, int B, int Hq, int Hkv, int N,
    int L, int S, int T, float sl2, int wg_per_bk, int sitems, int per_xcd) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[TfLds<D>::BYTES];
  const int nst = 8 * per_xcd;
  if ((int)blockIdx.x < nst) {
    using C = TsCfg<D>;
    taylor_state_item<D>(K, V, M0, z0, M_S, z_S, lens, Hkv, N, wg_per_bk, sitems, per_xcd, (int)blockIdx.x,
                         reinterpret_cast<__bf16 (*)[(D + 1) * C::TSTR]>(lds),
                         reinterpret_cast<__bf16 (*)[D * C::TSTR]>(lds + 2 * (D + 1) * C::TSTR * sizeof(__bf16)));
  } else {
    using C = TaCfg<D>;
    taylor_attn_item<D>(Q, K, V, beta, O, lse, lens, num0, den0, B, Hq, Hkv, N, L, S, T, sl2, (int)blockIdx.x - nst,
                        reinterpret_cast<__bf16 (*)[C::KTILE]>(lds),
                        reinterpret_cast<__bf16 (*)[C::TTILE]>(lds + 2 * C::KTILE * sizeof(__bf16)));
  }
}

// The kernel form costs 4 d per earlier key per query, so its work grows as
// N^2; the state sweep (fp32 vector kernels) costs about 4 D' d per token on a
// unit some ten times slower per flop.  Up to N = 16 D' tokens (66576 at
// d = 64, 264208 at d = 128) the kernel form is the cheaper one.
bool taylor_mfma_supported(const Geometry& g) {
  return g.fmap == 1 && g.dtype == 1 && (g.D == 64 || g.D == 128) &&
         (long long)g.N <= 16LL * (long long)taylor_dim(g.D);
}

size_t taylor_mfma_m0_bytes(const Geometry& g) {
  const size_t rows = (size_t)g.B * g.Hq * g.N;
  return ((rows * g.D * 4 + 255) / 256) * 256 + ((rows * 4 + 255) / 256) * 256;
}

hipError_t launch_taylor_mfma(const Geometry& g, const void* Q, const void* K, const void* V,
                              const float* beta, const float* M0, const float* z0, void* O, float* M_S, float* z_S,
                              float* lse, void* m0ws, hipStream_t st) {
  if (!taylor_mfma_supported(g)) return hipErrorInvalidValue;
  if ((M0 == nullptr) != (z0 == nullptr) || (M0 && !m0ws)) return hipErrorInvalidValue;
  float* num0 = nullptr;
  float* den0 = nullptr;
  if (M0) {
    const size_t rows = (size_t)g.B * g.Hq * g.N;
    num0 = static_cast<float*>(m0ws);
    den0 = reinterpret_cast<float*>(static_cast<char*>(m0ws) + ((rows * g.D * 4 + 255) / 256) * 256);
    const int tiles = (g.N + 255) / 256;
    const long long wgs = (long long)g.B * g.Hq * tiles;
    if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
#define TM_ARGS static_cast<const __bf16*>(Q), M0, z0, num0, den0, g.lens, g.Hq, g.Hkv, g.N, tiles
    if (g.D == 128) hipLaunchKernelGGL(taylor_m0_kernel<128>, dim3((unsigned)wgs), dim3(256), 0, st, TM_ARGS);
    else hipLaunchKernelGGL(taylor_m0_kernel<64>, dim3((unsigned)wgs), dim3(256), 0, st, TM_ARGS);
#undef TM_ARGS
  }
  const float sl2 = 1.4426950408889634f / sqrtf((float)g.D);
  const int T = (g.L + 63) / 64;
  const long long items = (long long)g.S * g.B * g.Hq * T;
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  const int wg_per_bk = g.D / 32 * 4 * (g.D / 64) + 1;   // pair workgroups + the linear one
  const long long sitems = (long long)g.B * g.Hkv * wg_per_bk;
  if (sitems > 0x7fffffffLL - 8) return hipErrorInvalidValue;
  const int per_xcd = (int)((sitems + 7) / 8);
  if (items + 8LL * per_xcd > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(items + 8LL * per_xcd));
#define TF_ARGS static_cast<const __bf16*>(Q), static_cast<const __bf16*>(K), static_cast<const __bf16*>(V), \
                beta, M0, z0, num0, den0, static_cast<__bf16*>(O), lse, M_S, z_S, g.lens, g.B, g.Hq, g.Hkv, g.N, \
                g.L, g.S, T, sl2, wg_per_bk, (int)sitems, per_xcd
  if (g.D == 128) hipLaunchKernelGGL(taylor_fwd_kernel<128>, grid, dim3(256), 0, st, TF_ARGS);
  else hipLaunchKernelGGL(taylor_fwd_kernel<64>, grid, dim3(256), 0, st, TF_ARGS);
#undef TF_ARGS
  return hipGetLastError();
}

}  // namespace infini
