// bf16 matrix-core forward of the Infini-attention segment kernel (gfx950).
//
// One workgroup = 8 waves = 256 query rows (head_dim 128; 4 waves = 128 rows
// for head_dim 64) of one (batch, query head, segment); each wave owns 32
// query rows, and all waves share each staged K/V tile.  A workgroup attends
// two such query tiles, p and nqt-1-p, one after the other, so that all
// workgroups walk the same number of key tiles.  Per 64-key tile:
//   S^T = K Q^T          v_mfma_f32_32x32x16_bf16, K from LDS, Q^T in registers
//   online softmax       base-2, row max/sum inside the lane plus one swap with
//                        the lane 32 apart (page "Context Memorization for
//                        Efficient Long Context Generation", section "방법론":
//                        attention states over key sub-blocks merge exactly)
//   O^T += V^T P^T       P^T straight from the S^T accumulators (no LDS trip);
//                        V^T staged transposed in LDS, its columns permuted so
//                        that each operand is one 16-byte read
// Working on the transposed products makes every lane own one query row, so
// the softmax statistics need no cross-lane reduction beyond one exchange.
//
// Epilogue (page "Hugging Face Infini-Attention 재현 분석", section
// "Infini-Attention 메커니즘", steps Memory Retrieval and Integration):
//   A_mem^T = M_{s-1}^T sigma(Q)^T   on the matrix cores, M^T (bf16) staged in
//                                    LDS through the free K/V staging registers
//   den     = sigma(Q) z_{s-1} + eps  fp32 dot per lane
//   O       = g A_mem + (1 - g) A_dot, rounded once to bf16
//
// Layout of the per-lane MFMA operands (gfx950, 32x32x16 bf16): A lane l holds
// row l%32, k = 8(l/32)..+7; B lane l holds column l%32, same k; the C/D lane l
// holds column l%32, rows 8(r/4) + 4(l/32) + r%4 for r = 0..15.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace infini {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int D>
struct FwdCfg {
  static constexpr int BM = D == 128 ? 256 : 128;   // query rows per workgroup
  static constexpr int WM = 32;           // query rows per wave
  static constexpr int NW = BM / WM;      // waves per workgroup
  static constexpr int NT = NW * 64;      // threads per workgroup
  static constexpr int BN = 64;           // keys per tile
  static constexpr int KS = D / 16;       // MFMA k-steps over head_dim
  static constexpr int DB = D / 32;       // 32-row blocks of head_dim
  static constexpr int KSTR = D + 8;      // K tile row stride (elements); 16-byte aligned rows
  static constexpr int VSTR = BN + 8;     // V^T tile row stride; 16-byte aligned rows
  static constexpr int KTILE = BN * KSTR;
  static constexpr int VTILE = D * VSTR;
  static constexpr int KPT = BN * D / 8 / NT;   // keys per thread when staging V^T
  static constexpr int CPT = BN * D / 8 / NT;   // 16-byte K chunks per thread per tile
  static constexpr int MSTR = D + 8;      // M^T stage row stride
  static constexpr int BUF = KTILE + VTILE;
  static constexpr int MT = 2 * BUF;      // M^T region, after the two tile buffers
  static constexpr int LDS_ELEMS = 2 * BUF + D * D;
};

// max / sum of x over lanes l and l^32 (v_permlane32_swap exchanges the two
// wave halves; the pair it returns holds both values in every lane).
__device__ __forceinline__ float pair_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// GROUPED: one launch for the segments of several calls of the same shape
// (spc segments each); segment sl of the launch is segment sl % spc of call
// sl / spc, whose tensors `tab` holds.  The published states (MsnapT, zsnap)
// are those of one memory phase over all the launch's segments.
template <int D, bool GROUPED>
__global__ __launch_bounds__(FwdCfg<D>::NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_mfma_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                     const __bf16* __restrict__ V, const float* __restrict__ beta,
                     const __bf16* __restrict__ MsnapT, const float* __restrict__ zsnap,
                     __bf16* __restrict__ O, float* __restrict__ lse,
                     int Hq, int Hkv, int N, int L, int s_begin, int nseg, int nqt, float sl2,
                     FwdCallTable tab, int spc, const int* __restrict__ lens) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 smem[C::LDS_ELEMS];
  __shared__ __attribute__((aligned(16))) float zs[D];

  // ---- work decode: each XCD (workgroups are dealt round-robin to 8 XCDs)
  // takes a contiguous range of work so that the query heads and tiles that
  // share one K/V segment run on the same L2.
  const int nwg = gridDim.x;
  int work = blockIdx.x;
  if ((nwg & 7) == 0) work = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  const int G = Hq / Hkv;
  // Each workgroup attends two query tiles of one (batch, head, segment),
  // nqt - 1 - p and p, so every workgroup walks the same number of key tiles
  // (the middle tile of an odd nqt goes alone).
  const int npair = (nqt + 1) / 2;
  const int per_group = G * npair;
  const int grp = work / per_group;
  const int rem = work % per_group;
  const int pr = rem / G;
  const int h_in = rem % G;
  const int sl = grp % nseg;
  const int bk = grp / nseg;                  // b * Hkv + kvh
  const int b = bk / Hkv, kvh = bk % Hkv;
  const int h = kvh * G + h_in;
  int s = s_begin + sl;                       // segment within its call
  if constexpr (GROUPED) {
    const int c = sl / spc;
    s = sl % spc;
    Q = tab.Q[c]; K = tab.K[c]; V = tab.V[c]; O = tab.O[c];
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 31, hh = lane >> 5;
  // waves w and w + 4 share a SIMD: they take row blocks w and 7 - w, so
  // that each SIMD's pair attends to the same number of diagonal tiles
  const int rblk = (C::NW == 8 && wave >= 4) ? 11 - wave : wave;
  const size_t qbase = (((size_t)b * Hq + h) * N + (size_t)s * L) * D;
  const size_t kvbase = (((size_t)b * Hkv + kvh) * N + (size_t)s * L) * D;
  // rows and keys of this segment: the last may be short, and in a
  // variable-length batch the segment may lie past its sequence's end
  const int Ls = min(L, seq_len_of(lens, b, N) - s * L);
  // query tiles of this workgroup that hold rows of the segment (a short
  // segment may end before them); the shorter one first, so that the longer
  // one's first key tiles are still in L2 when it reads them
  const int qtA = pr, qtB = nqt - 1 - pr;
  int nq = 0;
  if (qtA * C::BM < Ls) nq = (qtB != qtA && qtB * C::BM < Ls) ? 2 : 1;
  if (nq == 0) return;
  auto tiles_of = [&](int qt) { return (min(Ls, qt * C::BM + C::BM) + C::BN - 1) / C::BN; };
  const int nA = tiles_of(qtA);
  const int nsteps = nA + (nq > 1 ? tiles_of(qtB) : 0);   // key tiles of both query tiles, in order
  auto kofs = [&](int i) { return (i < nA ? i : i - nA) * C::BN; };

  // ---- Q^T operand of a query tile in registers for its whole key loop
  bf16x8_t qreg[C::KS];
  auto load_q = [&](int qt) {
    const int r = qt * C::BM + rblk * C::WM + lq;
    const bool ok = r < Ls;
    const __bf16* qp = Q + qbase + (size_t)(ok ? r : 0) * D + hh * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qp + ks * 16);
      qreg[ks] = ok ? v : bf16x8_t{};
    }
  };
  load_q(qtA);
  int q0 = 0, qrow = 0;   // wave's first row and this lane's query row in the current query tile

  // ---- global -> register staging of K and V tiles
  //
  // LDS holds two (K, V^T) buffers; tile j computes from buffer j & 1 while
  // tile j + 1, loaded into registers during tile j, is stored into the other
  // buffer at its end (one barrier per tile).
  bf16x8_t kst[C::CPT], vst[C::KPT];
  // V^T staging: consecutive lanes take consecutive key groups so that the
  // transposed LDS stores of a 16-lane group hit distinct banks.
  constexpr int NKG = C::BN / C::KPT;
  const int vkg = tid % NKG, vdc = tid / NKG;
  // Per-lane element offsets inside a tile are fixed; each tile adds a
  // workgroup-uniform row offset.  Keys past the segment end (only in the last
  // tile of a ragged segment) are clamped to its last row: finite values that
  // the score mask removes (K) or that meet a zero probability (V).
  const __bf16* Kseg = K + kvbase;
  const __bf16* Vseg = V + kvbase;
  // K chunk i of this thread: row krow0 + i * KRS, columns kcol .. kcol + 7
  constexpr int KRS = C::NT / (D / 8);
  const int krow0 = tid / (D / 8), kcol = (tid % (D / 8)) * 8;
  auto load_tile = [&](int k0) {
    const __bf16* kt = Kseg + (size_t)k0 * D + krow0 * D + kcol;
    const __bf16* vt = Vseg + (size_t)k0 * D;
    if (k0 + C::BN <= Ls) {
#pragma unroll
      for (int i = 0; i < C::CPT; ++i) kst[i] = *reinterpret_cast<const bf16x8_t*>(kt + i * KRS * D);
#pragma unroll
      for (int i = 0; i < C::KPT; ++i)
        vst[i] = *reinterpret_cast<const bf16x8_t*>(vt + (vkg * C::KPT + i) * D + vdc * 8);
    } else {
#pragma unroll
      for (int i = 0; i < C::CPT; ++i) {
        const int key = min(k0 + krow0 + i * KRS, Ls - 1);
        kst[i] = *reinterpret_cast<const bf16x8_t*>(Kseg + (size_t)key * D + kcol);
      }
#pragma unroll
      for (int i = 0; i < C::KPT; ++i) {
        const int key = min(k0 + vkg * C::KPT + i, Ls - 1);
        vst[i] = *reinterpret_cast<const bf16x8_t*>(Vseg + (size_t)key * D + vdc * 8);
      }
    }
  };
  // V^T columns hold the keys of each 16-key group with index bits 2 and 3
  // swapped, so that the 8 keys one lane's PV operand needs (see below) are
  // contiguous: one 16-byte LDS read per MFMA.
  auto vcol = [](int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); };
  auto store_tile = [&](int buf) {
    __bf16* Ks = smem + buf * C::BUF;
    __bf16* Vt = Ks + C::KTILE;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i)
      *reinterpret_cast<bf16x8_t*>(Ks + (krow0 + i * KRS) * C::KSTR + kcol) = kst[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16* dst = Vt + (vdc * 8 + e) * C::VSTR + vcol(vkg * C::KPT);
      if constexpr (C::KPT == 4) {
        bf16x4_t w = {vst[0][e], vst[1][e], vst[2][e], vst[3][e]};
        *reinterpret_cast<bf16x4_t*>(dst) = w;
      } else {
        bf16x2_t w = {vst[0][e], vst[1][e]};
        *reinterpret_cast<bf16x2_t*>(dst) = w;
      }
    }
  };

  // The retrieval operand M_{s-1}^T (bf16), shared by both query tiles, is
  // staged once, with the first K/V tile, into an LDS region of its own.
  // M^T rows are unpadded; 16-byte chunk c of row r sits at chunk
  // c ^ (r & 7), which keeps the epilogue's row reads conflict-free.
  constexpr int MPT = D * D / 8 / C::NT;  // 16-byte chunks of M^T per thread
  const __bf16* msrc = MsnapT + ((size_t)bk * nseg + sl) * D * D;
  const float* zsrc = zsnap + ((size_t)bk * nseg + sl) * D;
  // Chunk i of a thread in wave w covers 1 KB block i*NW + w, i.e. rows
  // (i*NW + w) * RPB + lane / (D/8); (row & 7) does not depend on i, so every
  // load of a lane is one base address plus a constant.
  constexpr int RPB = 64 / (D / 8);               // M^T rows per 1 KB block
  const int mrow0 = wave * RPB + lane / (D / 8);
  const __bf16* msrc0 = msrc + (size_t)mrow0 * D + (((lane % (D / 8)) ^ (mrow0 & 7)) * 8);
  __bf16* const Mts = smem + C::MT;

  f32x16_t oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16_t{};
  float m = -INFINITY, lpart = 0.f;

  // One 64-key tile for this wave's 32 rows.  Scores stay in the raw domain
  // until one FMA per element forms (s * scale * log2 e - m); the running max m
  // (scaled, base 2) only moves when a row's tile max exceeds it by more than
  // kRescaleSlack, so the accumulator rescale is skipped on almost every tile.
  // Any reference value gives the same normalised result; the slack bounds the
  // unnormalised terms by 2^kRescaleSlack.
  constexpr float kRescaleSlack = 8.f;
  const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};
  auto tile_step = [&](const __bf16* Ks, const __bf16* Vt, int k0, bool masked) {
    f32x16_t sacc[2];
    bf16x8_t ka[2][C::KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        ka[kb][ks] = *reinterpret_cast<const bf16x8_t*>(Ks + (kb * 32 + lq) * C::KSTR + ks * 16 + hh * 8);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kb][ks], qreg[ks], sacc[kb], 0, 0, 0);
    }
    // Issue order: the first block's K reads, then each of its products
    // beside one read of the second block, then the second block's products;
    // at most 15 reads are outstanding when a product waits for its operand.
    __builtin_amdgcn_sched_group_barrier(0x100, C::KS, 0);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, C::KS, 0);
    if (masked) {
      // element (kb, r) holds key k0 + 4hh + kb*32 + 8(r/4) + r%4
      const int lim = min(qrow, Ls - 1) - (k0 + 4 * hh);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) sacc[kb][r] = -INFINITY;
    }
    float mt = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
    mt = pair_max32(mt) * sl2;
    if (__builtin_amdgcn_ballot_w64(mt > m + kRescaleSlack)) {
      const float mn = fmaxf(m, mt);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      lpart *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
    }
    bf16x8_t pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        pb[kb][r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[kb][r], sl2, -m));
    // Row sum of the bf16 probabilities the PV product uses, two per v_dot2.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int x = 0; x < 4; ++x)
          lpart = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{pb[kb][t][2 * x], pb[kb][t][2 * x + 1]}, ones, lpart, false);
    // O^T += V^T P^T: k-slot q of half hh <-> key 16t + 8(q/4) + 4hh + q%4,
    // which is V^T column 16t + 8hh + q
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(Vt + (db * 32 + lq) * C::VSTR + kb * 32 + 16 * t + 8 * hh);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][t], oacc[db], 0, 0, 0);
        }
      }
    }
  };

  // The kernel arguments only the epilogue reads are brought into registers
  // here: a scalar load still in flight when the key loop starts would make
  // every tile's first LDS wait a full wait.
  asm volatile("" ::"s"(beta), "s"(O), "s"(lse), "s"(msrc));
  load_tile(0);
  {
    bf16x8_t mst[MPT];
#pragma unroll
    for (int i = 0; i < MPT; ++i) mst[i] = *reinterpret_cast<const bf16x8_t*>(msrc0 + (size_t)i * C::NW * RPB * D);
    // z_{s-1} has an LDS array of its own, written once before the first barrier
    if (wave < D / 64) zs[wave * 64 + lane] = zsrc[wave * 64 + lane];
    store_tile(0);
#pragma unroll
    for (int i = 0; i < MPT; ++i)
      *reinterpret_cast<bf16x8_t*>(Mts + (i * C::NW + wave) * 512 + lane * 8) = mst[i];
  }
  __syncthreads();
  if (nsteps > 1) load_tile(kofs(1));

  const float gt = sigmoid(beta[h]);
  int step = 0;   // key tiles walked so far (both query tiles); tile buffer step & 1
  for (int t = 0; t < nq; ++t) {
    const int qt = t == 0 ? qtA : qtB;
    q0 = qt * C::BM + rblk * C::WM;
    qrow = q0 + lq;
    const int ntiles = t == 0 ? nA : nsteps - nA;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16_t{};
    m = -INFINITY;
    lpart = 0.f;

    for (int j = 0; j < ntiles; ++j, ++step) {
      const int k0 = j * C::BN;
      const __bf16* Ks = smem + (step & 1) * C::BUF;
      const __bf16* Vt = Ks + C::KTILE;
      const bool active = k0 <= q0 + C::WM - 1 && q0 < Ls;
      const bool masked = (k0 + C::BN - 1 > q0) || (k0 + C::BN > Ls);
      if (active) {
        tile_step(Ks, Vt, k0, masked);
      }
      if (step + 1 < nsteps) store_tile((step + 1) & 1);
      __syncthreads();
      if (step + 2 < nsteps) load_tile(kofs(step + 2));
    }

    // ---- retrieval from M_{s-1}, z_{s-1} (staged in their own LDS) and the gate
    const float l = pair_sum32(lpart);

    bf16x8_t sq[C::KS];
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
    const float den = pair_sum32(dpart) + 1e-6f;
    f32x16_t nacc[C::DB];
#pragma unroll
    for (int cb = 0; cb < C::DB; ++cb) {
      nacc[cb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int r = cb * 32 + lq;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(Mts + r * D + (((ks * 2 + hh) ^ (r & 7)) * 8));
        nacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sq[ks], nacc[cb], 0, 0, 0);
      }
    }
    // the next query tile's Q rows arrive during this tile's output stores
    if (t + 1 < nq) load_q(qtB);
    const float wm = gt / den;
    const float wd = (1.f - gt) / l;
    if (qrow < Ls) {
      __bf16* op = O + qbase + (size_t)qrow * D;
#pragma unroll
      for (int cb = 0; cb < C::DB; ++cb) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          bf16x4_t w;
#pragma unroll
          for (int x = 0; x < 4; ++x) w[x] = (__bf16)(wm * nacc[cb][4 * u + x] + wd * oacc[cb][4 * u + x]);
          *reinterpret_cast<bf16x4_t*>(op + cb * 32 + 8 * u + 4 * hh) = w;
        }
      }
      if (lse && hh == 0)
        lse[((size_t)b * Hq + h) * N + (size_t)s * L + qrow] = (m + __log2f(l)) * 0.69314718055994531f;
    }
  }
}

template <int D>
static hipError_t fwd_mfma_t(const Geometry& g, const void* Q, const void* K, const void* V,
                             const float* beta, const void* MsnapT, const float* zsnap, void* O,
                             float* lse, int s_begin, int s_end, hipStream_t st) {
  const int nseg = s_end - s_begin;
  const int nqt = (g.L + FwdCfg<D>::BM - 1) / FwdCfg<D>::BM;
  const long long nwg = (long long)g.B * g.Hq * nseg * ((nqt + 1) / 2);
  if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL((fwd_mfma_kernel<D, false>), dim3((unsigned)nwg), dim3(FwdCfg<D>::NT), 0, st,
                     static_cast<const __bf16*>(Q), static_cast<const __bf16*>(K),
                     static_cast<const __bf16*>(V), beta, static_cast<const __bf16*>(MsnapT), zsnap,
                     static_cast<__bf16*>(O), lse, g.Hq, g.Hkv, g.N, g.L, s_begin, nseg, nqt, sl2,
                     FwdCallTable{}, 1, g.lens);
  return hipGetLastError();
}

template <int D>
static hipError_t fwd_mfma_group_t(const Geometry& g, const FwdCallTable& tab, int ncalls, const float* beta,
                                   const void* MsnapT, const float* zsnap, hipStream_t st) {
  const int nseg = ncalls * g.S;
  const int nqt = (g.L + FwdCfg<D>::BM - 1) / FwdCfg<D>::BM;
  const long long nwg = (long long)g.B * g.Hq * nseg * ((nqt + 1) / 2);
  if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL((fwd_mfma_kernel<D, true>), dim3((unsigned)nwg), dim3(FwdCfg<D>::NT), 0, st,
                     nullptr, nullptr, nullptr, beta, static_cast<const __bf16*>(MsnapT), zsnap, nullptr,
                     nullptr, g.Hq, g.Hkv, g.N, g.L, 0, nseg, nqt, sl2, tab, g.S, nullptr);
  return hipGetLastError();
}

hipError_t launch_fwd_mfma_group(const Geometry& g, const FwdCallTable& tab, int ncalls, const float* beta,
                                 const void* MsnapT, const float* zsnap, hipStream_t st) {
  if (g.dtype != 1 || ncalls < 1 || ncalls > kFwdMaxGroup) return hipErrorInvalidValue;
  if (g.D == 128) return fwd_mfma_group_t<128>(g, tab, ncalls, beta, MsnapT, zsnap, st);
  if (g.D == 64) return fwd_mfma_group_t<64>(g, tab, ncalls, beta, MsnapT, zsnap, st);
  return hipErrorInvalidValue;
}

bool fwd_mfma_supported(const Geometry& g) { return g.fmap == 0 && g.dtype == 1 && (g.D == 64 || g.D == 128); }

hipError_t launch_fwd_mfma(const Geometry& g, const void* Q, const void* K, const void* V,
                           const float* beta, const void* MsnapT, const float* zsnap, void* O,
                           float* lse, int s_begin, int s_end, hipStream_t st) {
  if (g.dtype != 1) return hipErrorInvalidValue;
  if (g.D == 128) return fwd_mfma_t<128>(g, Q, K, V, beta, MsnapT, zsnap, O, lse, s_begin, s_end, st);
  if (g.D == 64) return fwd_mfma_t<64>(g, Q, K, V, beta, MsnapT, zsnap, O, lse, s_begin, s_end, st);
  return hipErrorInvalidValue;
}

}  // namespace infini
