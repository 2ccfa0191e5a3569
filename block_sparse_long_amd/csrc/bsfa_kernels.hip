// Exact-score-gated block-sparse causal prefill attention for gfx950 (MI355X).
//
// The method ("Block Sparse Flash Attention", paper notes, Method > Key Designs 2 and 3): every
// causally visible QK^T tile is computed exactly; the tile's maximum scaled score s_max decides
// whether an off-diagonal key block is kept (s_max >= T) or skipped. A skipped block loads no
// V, computes no exponentials and leaves the online-softmax state alone; the diagonal region
// always runs with the causal mask; the output is renormalised over the kept blocks. The
// relative gate ("Skipping attention blocks was the easy part", BLASST blog, "Vote, then skip")
// keeps a block iff some row's block max is within ln(lambda) of its running max.
//
// Mapping onto CDNA4:
//   * One wavefront owns 64 query rows of one head. Scores are produced transposed,
//     S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T resident in VGPRs),
//     so each lane holds 32 scores of each of its 2 rows: the row max is an in-lane max3 chain
//     plus one cross-half exchange, and the exponentials stay in the lanes that produced them.
//   * O^T = V^T P^T: P^T is the MFMA B operand straight from the softmax registers; V^T comes
//     from LDS, where V tiles are stored transposed with a key permutation that matches the
//     lane order of P (16 contiguous bytes per operand).
//   * A workgroup is 4 waves (256 query rows: 2 heads x 128 rows under GQA, or 4 x 64): each
//     K/V tile is staged in LDS once and read by every wave. K and V are double-buffered.
//   * QK of tile t+1 is issued before the softmax of tile t, so the gate statistics of tile
//     t+1 reach LDS before the one barrier of the iteration; V_t is fetched only when some
//     head of the workgroup keeps tile t, and is written to LDS behind the softmax.
//   * Workgroups are ordered heaviest query block first, and (when the unit count allows)
//     all query blocks of one KV head go to the same XCD so their K/V stream shares its L2.
#include "bsfa_internal.h"

#include <math.h>

namespace bsfa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int BK = kBlockK;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Position of key k (0..63) inside a transposed V row: within each group of 16 keys, the 8
// keys one lane half feeds to one MFMA k-step (keys 4h..4h+3 and 8+4h..8+4h+3 of the group)
// become contiguous, matching the order in which the P^T operand holds them.
__device__ __forceinline__ int vpos(int k) {
  return (k & ~15) | (((k >> 2) & 1) << 3) | (((k >> 3) & 1) << 2) | (k & 3);
}

template <int D>
struct Tile {
  static constexpr int KSTR = D + 8;        // K tile row stride in LDS (bf16), 16-byte padded
  static constexpr int VSTR = BK + 8;       // V^T tile row stride in LDS (bf16)
  static constexpr int KS = D / 16;         // QK k-steps over d
  static constexpr int MD = D / 32;         // PV M-blocks over d
  static constexpr int CPR = D / 8;         // 16-byte chunks per K/V row
};

// K tile: global [64 keys][D] -> registers -> LDS [key][D] (padded rows).
template <int D, int NT>
struct KStage {
  static constexpr int PER = BK * Tile<D>::CPR / NT;
  uint4 r[PER];
  __device__ __forceinline__ void load(const __bf16* base, long long kst, int nvalid, int tid) {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int c = tid + it * NT;
      const int row = c / Tile<D>::CPR, col = c % Tile<D>::CPR;
      const uint4 x = *reinterpret_cast<const uint4*>(base + min(row, nvalid - 1) * kst + col * 8);
      r[it] = row < nvalid ? x : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(__bf16* sk, int tid) const {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int c = tid + it * NT;
      const int row = c / Tile<D>::CPR, col = c % Tile<D>::CPR;
      *reinterpret_cast<uint4*>(sk + row * Tile<D>::KSTR + col * 8) = r[it];
    }
  }
};

// V tile: global [64 keys][D] -> registers -> LDS V^T [D][64 permuted keys]. Each work item is
// a key pair (2kp, 2kp+1) times 8 dims; the pair lands in one 32-bit LDS word per dim.
template <int D, int NT>
struct VStage {
  static constexpr int PER = 32 * Tile<D>::CPR / NT;
  uint4 a[PER], b[PER];
  __device__ __forceinline__ void load(const __bf16* base, long long vst, int nvalid, int tid) {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int item = tid + it * NT;
      const int kp = item & 31, dc = item >> 5;
      const int k0 = 2 * kp;
      const uint4 xa = *reinterpret_cast<const uint4*>(base + min(k0, nvalid - 1) * vst + dc * 8);
      const uint4 xb =
          *reinterpret_cast<const uint4*>(base + min(k0 + 1, nvalid - 1) * vst + dc * 8);
      a[it] = k0 < nvalid ? xa : make_uint4(0, 0, 0, 0);
      b[it] = k0 + 1 < nvalid ? xb : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(__bf16* sv, int tid) const {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int item = tid + it * NT;
      const int kp = item & 31, dc = item >> 5;
      const int pos = vpos(2 * kp);
      const uint32_t aw[4] = {a[it].x, a[it].y, a[it].z, a[it].w};
      const uint32_t bw[4] = {b[it].x, b[it].y, b[it].z, b[it].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (aw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        const uint32_t hi = (bw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        *reinterpret_cast<uint32_t*>(sv + (dc * 8 + e) * Tile<D>::VSTR + pos) = lo | (hi << 16);
      }
    }
  }
};

// S^T[key][row] for one 64-key tile and the wave's 64 rows: s[mb][nb] holds keys
// mb*32 + 8*(v/4) + 4*(lane/32) + v%4 and row nb*32 + lane%32 in element v. Both operands come
// from LDS: K (A operand) from the shared tile, Q^T (B operand) from the wave's own Q rows.
template <int D>
__device__ __forceinline__ void qk_tile(const __bf16* sk, const __bf16* sq, f32x16 (&s)[2][2],
                                        int lane) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[mb][nb][v] = 0.f;
  const int rl = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < Tile<D>::KS; ++ks) {
    bf16x8 qb[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      qb[nb] = *reinterpret_cast<const bf16x8*>(sq + (nb * 32 + rl) * Tile<D>::KSTR + ks * 16 +
                                                8 * hh);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(
          sk + (mb * 32 + rl) * Tile<D>::KSTR + ks * 16 + 8 * hh);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) s[mb][nb] = mfma32(a, qb[nb], s[mb][nb]);
    }
  }
}

// Same product with Q^T held in VGPRs (used where registers are plentiful).
template <int D>
__device__ __forceinline__ void qk_tile_regs(const __bf16* sk, const bf16x8 (&qf)[2][D / 16],
                                             f32x16 (&s)[2][2], int lane) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[mb][nb][v] = 0.f;
  const int rl = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < Tile<D>::KS; ++ks) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(
          sk + (mb * 32 + rl) * Tile<D>::KSTR + ks * 16 + 8 * hh);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) s[mb][nb] = mfma32(a, qf[nb][ks], s[mb][nb]);
    }
  }
}

template <int D>
__device__ __forceinline__ void load_q_regs(const __bf16* qbase, long long qst, int row0, int N,
                                            bf16x8 (&qf)[2][D / 16], int lane) {
  const int rl = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int row = row0 + nb * 32 + rl;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const uint4 x =
          *reinterpret_cast<const uint4*>(qbase + min(row, N - 1) * qst + ks * 16 + 8 * hh);
      const uint4 y = row < N ? x : make_uint4(0, 0, 0, 0);
      qf[nb][ks] = __builtin_bit_cast(bf16x8, y);
    }
  }
}

// Causal / ragged masking (when `masked`) and the per-row max over the 64 keys of the tile.
__device__ __forceinline__ void tile_rowmax(f32x16 (&s)[2][2], float (&rmax)[2], bool masked,
                                            int key0, int row0, int N, int lane) {
  const int rl = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int row = row0 + nb * 32 + rl;
    if (masked) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = key0 + mb * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (key > row || row >= N) s[mb][nb][v] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[mb][nb][v]);
    rmax[nb] = fmaxf(mx, __shfl_xor(mx, 32));
  }
}

// Online-softmax update for a kept tile (BLASST blog, "FlashAttention": running max m, sum l,
// accumulator O, rescale by exp(m_old - m_new)). The exponent reference mref moves only when a
// row's true max mt exceeds it by more than kLazy in the exp2 domain ("rescale ... when
// needed", paper notes, Key Designs 3): exponentials stay <= 2^kLazy, O/l is unchanged, and
// the O rescale (a VALU pass over the accumulators) becomes rare. mt is the exact running max
// the relative gate compares against. Writes P^T as bf16 MFMA B operands pb[nb][k-step].
constexpr float kLazy = 8.f;

template <int MD>
__device__ __forceinline__ void softmax_tile(const f32x16 (&s)[2][2], const float (&rmax)[2],
                                             float (&mt)[2], float (&mref)[2], float (&l)[2],
                                             f32x16 (&o)[MD][2], bf16x8 (&pb)[2][4], float c) {
  float mn[2];
  bool move = false;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    mn[nb] = fmaxf(mt[nb], rmax[nb]);
    mt[nb] = mn[nb];
    move |= (mn[nb] - mref[nb]) * c > kLazy;    // false for rows that see nothing (-inf - -inf)
  }
  if (__any(move)) {
    float alpha[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float mu = (mn[nb] == kNegInf) ? 0.f : mn[nb];
      alpha[nb] = __builtin_amdgcn_exp2f((mref[nb] - mu) * c);   // 0 on the first kept block
      mref[nb] = mu;
      l[nb] *= alpha[nb];
    }
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[md][nb][v] *= alpha[nb];
  }
  // l sums exactly the bf16 weights the PV product uses (two per v_dot2 against (1, 1)), so
  // O / l is a convex combination of V rows even though P is rounded for the MFMA.
  bf16x2 ones;
  ones[0] = (__bf16)1.f;
  ones[1] = (__bf16)1.f;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float off = -mref[nb] * c;
    float sum = 0.f;
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[ks2 >> 1][nb][(ks2 & 1) * 8 + e], c, off));
        const float p1 =
            __builtin_amdgcn_exp2f(fmaf(s[ks2 >> 1][nb][(ks2 & 1) * 8 + e + 1], c, off));
        bf16x2 pr;
        pr[0] = (__bf16)p0;
        pr[1] = (__bf16)p1;
        sum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, sum, false);
        pb[nb][ks2][e] = pr[0];
        pb[nb][ks2][e + 1] = pr[1];
      }
    }
    l[nb] += sum;
  }
}

template <int D>
__device__ __forceinline__ void pv_tile(const __bf16* sv, const bf16x8 (&pb)[2][4],
                                        f32x16 (&o)[D / 32][2], int lane) {
  const int rl = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int ks2 = 0; ks2 < 4; ++ks2) {
#pragma unroll
    for (int md = 0; md < Tile<D>::MD; ++md) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(
          sv + (md * 32 + rl) * Tile<D>::VSTR + 16 * ks2 + 8 * hh);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) o[md][nb] = mfma32(a, pb[nb][ks2], o[md][nb]);
    }
  }
}

struct Unit {
  int b, g, hg, i;
};

__device__ __forceinline__ Unit decode_unit(int L, int units, int nqb, int B, int Hkv,
                                            int xcd_map) {
  int i, u;
  if (xcd_map) {
    const int x = L & 7, s = L >> 3, upx = units >> 3;
    i = nqb - 1 - s / upx;
    u = (s % upx) * 8 + x;
  } else {
    i = nqb - 1 - L / units;
    u = L % units;
  }
  const int bh = u % (B * Hkv);
  Unit r;
  r.hg = u / (B * Hkv);
  r.b = bh / Hkv;
  r.g = bh % Hkv;
  r.i = i;
  return r;
}

// The wave's 64 query rows -> LDS [row][D] (padded rows); rows past N are zero.
template <int D>
__device__ __forceinline__ void stage_q(const __bf16* qbase, long long qst, int row0, int N,
                                        __bf16* sq, int lane) {
  constexpr int CPR = Tile<D>::CPR;
#pragma unroll
  for (int it = 0; it < 64 * CPR / 64; ++it) {
    const int c = lane + it * 64;
    const int r = c / CPR, col = c % CPR;
    const int row = row0 + r;
    const uint4 x = *reinterpret_cast<const uint4*>(qbase + min(row, N - 1) * qst + col * 8);
    *reinterpret_cast<uint4*>(sq + r * Tile<D>::KSTR + col * 8) =
        row < N ? x : make_uint4(0, 0, 0, 0);
  }
}

template <int D, int BQ, int NW, int GATE>
__global__ __launch_bounds__(NW * 64, 1) void prefill_kernel(PrefillArgs a) {
  constexpr int NT = NW * 64;
  constexpr int WPH = BQ / 64;             // waves per head
  constexpr int HPW = NW / WPH;            // heads per workgroup
  constexpr int MD = Tile<D>::MD;
  constexpr bool kGated = GATE != kDense;

  __shared__ __attribute__((aligned(16))) __bf16 sQ[NW][64 * Tile<D>::KSTR];
  __shared__ __attribute__((aligned(16))) __bf16 sK[2][BK * Tile<D>::KSTR];
  __shared__ __attribute__((aligned(16))) __bf16 sV[2][D * Tile<D>::VSTR];
  __shared__ float sGate[2][NW];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hw = w / WPH, rw = w % WPH;
  const Unit un = decode_unit(blockIdx.x, a.units, a.nqb, a.B, a.Hkv, a.xcd_map);
  const int b = un.b, g = un.g, i = un.i;
  const int h0 = g * a.G + un.hg * HPW;
  const int h = h0 + hw;
  const int N = a.N;
  const int row0 = i * BQ + rw * 64;
  const int n_off = (i * BQ) / BK;
  const int n_end = (min((i + 1) * BQ, N) - 1) / BK + 1;
  const bool ragged_rows = (i + 1) * BQ > N;
  const bool want_stat = kGated || a.dbg != nullptr;
  const bool head_leader = (rw == 0) && (lane == 0);

  const __bf16* Qb = static_cast<const __bf16*>(a.q) + b * a.qs[0] + h * a.qs[2];
  const __bf16* Kb = static_cast<const __bf16*>(a.k) + b * a.ks[0] + g * a.ks[2];
  const __bf16* Vb = static_cast<const __bf16*>(a.v) + b * a.vs[0] + g * a.vs[2];

  float thr[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    if (GATE == kAbsolute)
      thr[hh] = a.thr[(h0 + hh) * a.t_len + min(i, a.t_len - 1)];
    else if (GATE == kRelative)
      thr[hh] = a.log_lambda;
    else
      thr[hh] = kNegInf;
  }

  stage_q<D>(Qb, a.qs[1], row0, N, sQ[w], lane);
  const __bf16* sq = sQ[w];

  // mt: true running row max (over kept blocks); mref: exponent reference (lazy)
  float mt[2] = {kNegInf, kNegInf}, mref[2] = {kNegInf, kNegInf}, l[2] = {0.f, 0.f};
  f32x16 o[MD][2];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[md][nb][v] = 0.f;

  KStage<D, NT> kst;
  VStage<D, NT> vst;

  auto key_valid = [&](int j) { return min(BK, N - j * BK); };
  auto tile_masked = [&](int j) { return j >= n_off || ragged_rows; };

  // Gate statistic of this wave for tile j (raw score units; the scale is applied at the
  // decision): s_max (ABSOLUTE, DENSE, and the diagonal region in every mode) or
  // max over rows of (rowmax - running max) (RELATIVE, off-diagonal).
  auto publish = [&](int j, const float (&rmax)[2]) {
    float st;
    if (GATE == kRelative && j < n_off) {
      float x = kNegInf;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int row = row0 + nb * 32 + (lane & 31);
        const float d = rmax[nb] - mt[nb];
        x = fmaxf(x, row < N ? d : kNegInf);
      }
      st = wave_max(x);
    } else {
      st = wave_max(fmaxf(rmax[0], rmax[1]));
    }
    if (lane == 0) sGate[j & 1][w] = st;
  };

  // ---- prologue: K_0 staged, S_0 computed and published ----
  kst.load(Kb, a.ks[1], key_valid(0), tid);
  kst.store(sK[0], tid);
  __syncthreads();
  if (n_end > 1) kst.load(Kb + (long long)BK * a.ks[1], a.ks[1], key_valid(1), tid);
  f32x16 sc[2][2];
  float rc[2];
  qk_tile<D>(sK[0], sq, sc, lane);
  tile_rowmax(sc, rc, tile_masked(0), 0, row0, N, lane);
  if (want_stat) publish(0, rc);
  if (n_end > 1) kst.store(sK[1], tid);
  __syncthreads();

  int kept = 0;
  bool keep_prev = false;
  bf16x8 pbp[2][4];   // P of the previous kept tile, consumed by its PV in this iteration

  for (int t = 0; t < n_end; ++t) {
    // ---- decision for tile t (statistics visible since the last barrier) ----
    const bool diag = t >= n_off;
    bool mykeep = true, anyv = true;
    if (want_stat) {
      float hst[HPW];
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        float x = sGate[t & 1][hh * WPH];
#pragma unroll
        for (int r = 1; r < WPH; ++r) x = fmaxf(x, sGate[t & 1][hh * WPH + r]);
        hst[hh] = x * a.scale;
      }
      if (kGated && !diag) {
        anyv = false;
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          const bool k = hst[hh] >= thr[hh];
          anyv |= k;
          if (hh == hw) mykeep = k;
        }
      }
      if (head_leader) {
        if (!diag) kept += mykeep ? 1 : 0;
        if (a.dbg) a.dbg[(((long long)b * a.Hq + h) * a.nqb + i) * a.nkb + t] = hst[hw];
      }
    } else if (head_leader && !diag) {
      kept += 1;
    }

    // global loads for V_t (only if some head keeps tile t) and K_{t+2}; they land in LDS at
    // the end of the iteration
    if (anyv) vst.load(Vb + (long long)t * BK * a.vs[1], a.vs[1], key_valid(t), tid);
    if (t + 2 < n_end)
      kst.load(Kb + (long long)(t + 2) * BK * a.ks[1], a.ks[1], key_valid(t + 2), tid);

    // PV of the previous kept tile (MFMA) next to the exponentials of this one (VALU)
    if (keep_prev) pv_tile<D>(sV[(t - 1) & 1], pbp, o, lane);
    bf16x8 pbn[2][4];
    if (mykeep) softmax_tile<MD>(sc, rc, mt, mref, l, o, pbn, a.c_log2);

    // scores of the next tile reuse the registers of this one
    if (t + 1 < n_end) {
      qk_tile<D>(sK[(t + 1) & 1], sq, sc, lane);
      tile_rowmax(sc, rc, tile_masked(t + 1), (t + 1) * BK, row0, N, lane);
      if (want_stat) publish(t + 1, rc);
    }
    if (anyv) vst.store(sV[t & 1], tid);
    if (t + 2 < n_end) kst.store(sK[t & 1], tid);
    __syncthreads();

    if (mykeep) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int ks2 = 0; ks2 < 4; ++ks2) pbp[nb][ks2] = pbn[nb][ks2];
    }
    keep_prev = mykeep;
  }
  if (keep_prev) pv_tile<D>(sV[(n_end - 1) & 1], pbp, o, lane);

  // ---- epilogue: O / l (renormalised over kept + diagonal), kept counts ----
  const int rl = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float lt = l[nb] + __shfl_xor(l[nb], 32);
    const float inv = 1.f / lt;
    const int row = row0 + nb * 32 + rl;
    if (row < N) {
      const long long base = b * a.os[0] + (long long)row * a.os[1] + h * a.os[2];
#pragma unroll
      for (int md = 0; md < MD; ++md) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = md * 32 + 8 * q4 + 4 * hh;
          const float x0 = o[md][nb][4 * q4 + 0] * inv, x1 = o[md][nb][4 * q4 + 1] * inv;
          const float x2 = o[md][nb][4 * q4 + 2] * inv, x3 = o[md][nb][4 * q4 + 3] * inv;
          if (a.out_fp32) {
            *reinterpret_cast<float4*>(static_cast<float*>(a.o) + base + d0) =
                make_float4(x0, x1, x2, x3);
          } else {
            typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
            bf16x4 y;
            y[0] = (__bf16)x0;
            y[1] = (__bf16)x1;
            y[2] = (__bf16)x2;
            y[3] = (__bf16)x3;
            *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.o) + base + d0) = y;
          }
        }
      }
    }
  }
  if (head_leader) {
    if (a.kept_counts) a.kept_counts[((long long)b * a.Hq + h) * a.nqb + i] = kept;
    if (a.kept_total) atomicAdd(a.kept_total, (unsigned long long)kept);
  }
}

// Calibration: per (b, h, i) the off-diagonal block maxima, then the k-th highest per budget.
template <int D, int BQ, int NW>
__global__ __launch_bounds__(NW * 64, 1) void calibrate_kernel(CalibArgs a) {
  constexpr int NT = NW * 64;
  constexpr int WPH = BQ / 64;
  constexpr int HPW = NW / WPH;
  constexpr int MAXJ = kCalibMaxKeyBlocks;

  __shared__ __attribute__((aligned(16))) __bf16 sK[2][BK * Tile<D>::KSTR];
  __shared__ float sW[NW][MAXJ];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hw = w / WPH, rw = w % WPH;
  const Unit un = decode_unit(blockIdx.x, a.units, a.nqb, a.B, a.Hkv, a.xcd_map);
  const int b = un.b, g = un.g, i = un.i;
  const int h0 = g * a.G + un.hg * HPW;
  const int h = h0 + hw;
  const int N = a.N;
  const int row0 = i * BQ + rw * 64;
  const int n_off = (i * BQ) / BK;
  const bool ragged_rows = (i + 1) * BQ > N;

  if (n_off > 0) {
    const __bf16* Qb = static_cast<const __bf16*>(a.q) + b * a.qs[0] + h * a.qs[2];
    const __bf16* Kb = static_cast<const __bf16*>(a.k) + b * a.ks[0] + g * a.ks[2];
    bf16x8 qf[2][D / 16];
    load_q_regs<D>(Qb, a.qs[1], row0, N, qf, lane);
    KStage<D, NT> kst;
    kst.load(Kb, a.ks[1], BK, tid);
    kst.store(sK[0], tid);
    __syncthreads();
    for (int t = 0; t < n_off; ++t) {
      if (t + 1 < n_off) kst.load(Kb + (long long)(t + 1) * BK * a.ks[1], a.ks[1], BK, tid);
      f32x16 s[2][2];
      float rmax[2];
      qk_tile_regs<D>(sK[t & 1], qf, s, lane);
      tile_rowmax(s, rmax, ragged_rows, t * BK, row0, N, lane);
      const float st = wave_max(fmaxf(rmax[0], rmax[1]));
      if (lane == 0) sW[w][t] = st * a.scale;
      if (t + 1 < n_off) kst.store(sK[(t + 1) & 1], tid);
      __syncthreads();
    }
  }
  // merge the waves of each head into the list of its first wave; pad to a power of two
  int P = 1;
  while (P < n_off) P <<= 1;
  for (int idx = tid; idx < HPW * P; idx += NT) {
    const int hh = idx / P, t = idx % P;
    float x = kNegInf;
    if (t < n_off) {
      x = sW[hh * WPH][t];
      for (int r = 1; r < WPH; ++r) x = fmaxf(x, sW[hh * WPH + r][t]);
    }
    sW[hh * WPH][t] = x;
  }
  __syncthreads();
  // ascending bitonic sort of each head's list
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int idx = tid; idx < HPW * P; idx += NT) {
        const int hh = idx / P, x = idx % P, y = x ^ j;
        if (y > x) {
          float* L = sW[hh * WPH];
          const float u = L[x], v = L[y];
          const bool asc = (x & k) == 0;
          if ((u > v) == asc) {
            L[x] = v;
            L[y] = u;
          }
        }
      }
      __syncthreads();
    }
  }
  if (rw == 0) {
    for (int kk = lane; kk < a.n_budgets; kk += 64) {
      const int kb = a.budgets[kk];
      const float r = (n_off >= kb) ? sW[w][P - kb] : kNegInf;
      a.kth[(((long long)kk * a.B + b) * a.Hq + h) * a.nqb + i] = r;
    }
  }
}

__global__ void zero_u64_kernel(unsigned long long* p) { *p = 0ull; }

template <int D, int BQ, int NW>
hipError_t launch_prefill_gate(const PrefillArgs& a, int gate, hipStream_t stream) {
  const dim3 grid(a.units * a.nqb), block(NW * 64);
  switch (gate) {
    case kDense:
      hipLaunchKernelGGL((prefill_kernel<D, BQ, NW, kDense>), grid, block, 0, stream, a);
      break;
    case kAbsolute:
      hipLaunchKernelGGL((prefill_kernel<D, BQ, NW, kAbsolute>), grid, block, 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((prefill_kernel<D, BQ, NW, kRelative>), grid, block, 0, stream, a);
      break;
  }
  return hipGetLastError();
}

template <int D, int BQ>
hipError_t launch_prefill_nw(const PrefillArgs& a, int nw, int gate, hipStream_t stream) {
  if (BQ == 64 && nw == 1) return launch_prefill_gate<D, BQ, (BQ == 64 ? 1 : 2)>(a, gate, stream);
  if (nw == 2) return launch_prefill_gate<D, BQ, 2>(a, gate, stream);
  return launch_prefill_gate<D, BQ, 4>(a, gate, stream);
}

template <int D, int BQ>
hipError_t launch_calib_nw(const CalibArgs& a, int nw, hipStream_t stream) {
  const dim3 grid(a.units * a.nqb);
  if (BQ == 64 && nw == 1) {
    constexpr int NW = BQ == 64 ? 1 : 2;
    hipLaunchKernelGGL((calibrate_kernel<D, BQ, NW>), grid, dim3(NW * 64), 0, stream, a);
  } else if (nw == 2) {
    hipLaunchKernelGGL((calibrate_kernel<D, BQ, 2>), grid, dim3(128), 0, stream, a);
  } else {
    hipLaunchKernelGGL((calibrate_kernel<D, BQ, 4>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

int waves_per_workgroup(int block_q, int group) {
  const int wph = block_q / 64;
  int hpw = 4 / wph;
  while (hpw > 1 && group % hpw != 0) hpw >>= 1;
  return hpw * wph;
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int block_q, int gate,
                          hipStream_t stream) {
  const int nw = waves_per_workgroup(block_q, a.G);
  if (head_dim == 128) {
    return block_q == 128 ? launch_prefill_nw<128, 128>(a, nw, gate, stream)
                          : launch_prefill_nw<128, 64>(a, nw, gate, stream);
  }
  return block_q == 128 ? launch_prefill_nw<64, 128>(a, nw, gate, stream)
                        : launch_prefill_nw<64, 64>(a, nw, gate, stream);
}

hipError_t launch_calibrate(const CalibArgs& a, int head_dim, int block_q, hipStream_t stream) {
  const int nw = waves_per_workgroup(block_q, a.G);
  if (head_dim == 128) {
    return block_q == 128 ? launch_calib_nw<128, 128>(a, nw, stream)
                          : launch_calib_nw<128, 64>(a, nw, stream);
  }
  return block_q == 128 ? launch_calib_nw<64, 128>(a, nw, stream)
                        : launch_calib_nw<64, 64>(a, nw, stream);
}

hipError_t launch_zero_u64(unsigned long long* p, hipStream_t stream) {
  hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(1), 0, stream, p);
  return hipGetLastError();
}

}  // namespace bsfa
