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

#include <type_traits>

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

// O^T += V^T P^T with the accumulator pinned to AGPRs (inline asm): the score MFMAs write
// VGPRs, which the softmax reads directly, while O, touched only by these MFMAs, the rare
// rescale and the epilogue, lives in the accumulation registers. The compiler cannot see
// inside the asm, so the hazards around it are resolved by hand:
//   * consecutive accumulations into the same full accumulator need no wait states;
//   * P (SrcB) is written by VALU: pv_operands_ready() puts wait states between the last such
//     write and the first MFMA, and keep_alive() holds P's registers until the block ends so
//     no VALU write can land in a register an issued MFMA is still reading;
//   * VALU access to O after these MFMAs goes through acc_ready(), which waits out the
//     longest MFMA-result latency first.
__device__ __forceinline__ void mfma_acc(f32x16& o, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(b));
}

__device__ __forceinline__ float bits_f(int x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ int f_bits(float x) { return __builtin_bit_cast(int, x); }

// max / sum of x over lanes l and l^32 (the two halves holding the same query row)
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(f_bits(x), f_bits(x), false, false);
  return fmaxf(bits_f(r[0]), bits_f(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(f_bits(x), f_bits(x), false, false);
  return bits_f(r[0]) + bits_f(r[1]);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return bits_f(__builtin_amdgcn_update_dpp(0, f_bits(x), CTRL, 0xf, 0xf, false));
}

// Wave-uniform max over the 64 lanes: a butterfly within each row of 16 lanes (DPP quad
// permutes, half-row and row mirrors), then the four row results through readlane.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));     // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp<0x4E>(x));     // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp<0x141>(x));    // row_half_mirror
  x = fmaxf(x, dpp<0x140>(x));    // row_mirror
  const float r0 = bits_f(__builtin_amdgcn_readlane(f_bits(x), 0));
  const float r1 = bits_f(__builtin_amdgcn_readlane(f_bits(x), 16));
  const float r2 = bits_f(__builtin_amdgcn_readlane(f_bits(x), 32));
  const float r3 = bits_f(__builtin_amdgcn_readlane(f_bits(x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

template <int D>
struct Tile {
  static constexpr int CPR = D / 8;         // 16-byte chunks of data per row (16 or 8)
  static constexpr int STR = D + 8;         // Q/K row stride in bf16 (one 16-byte pad chunk)
  static constexpr int STRV = D + 32;       // V row stride in bf16 (four pad chunks)
  static constexpr int KS = D / 16;         // QK k-steps over d
  static constexpr int MD = D / 32;         // PV M-blocks over d
};

// LDS tiles hold 64 rows of D bf16 plus padding, so that every fragment address is a per-lane
// base plus a compile-time offset, and the rows one read touches spread over the 64 banks:
//   * Q and K (row stride D + 8): a 16-byte operand read covers 16 consecutive rows per
//     16 lanes; rows start 4 banks apart, so the 16 reads tile all 64 banks.
//   * V (row stride D + 32): a transposing read covers 4 consecutive rows x 64 bytes per 32
//     lanes; rows start 16 banks apart, so the 4 row segments are disjoint.
template <int D>
__device__ __forceinline__ int elem_off(int r, int c) {
  return r * Tile<D>::STR + (c << 3);
}

// Direct global -> LDS copy of a 64-row tile with row stride STRIDE (bf16), 1 KB per
// instruction: lane l of instruction k fills padded chunk q = 64k + l (row q / CPS, column
// q % CPS) with the matching global chunk; pad chunks re-fetch the row's last chunk. Rows at or
// past `valid` re-read row valid - 1 (their scores are masked and their P weights are zero).
// Wave w of NW issues instructions k = w + NW*m for a fixed m range, so every wave runs the
// same straight-line code; instructions past the tile's chunk count land in the spare space of
// a buffer sized by tile_elems<STRIDE, NW>() and fetch clamped, valid addresses.
template <int STRIDE, int NW>
constexpr int tile_instr_per_wave() {
  return (STRIDE / 8 + NW - 1) / NW;       // 64 rows x STRIDE/8 chunks = STRIDE/8 instructions
}
template <int STRIDE, int NW>
constexpr int tile_elems() {
  return tile_instr_per_wave<STRIDE, NW>() * NW * 512;
}

template <int D, int STRIDE, int NW>
__device__ __forceinline__ void wg_copy_tile(const __bf16* gbase, long long gst, int valid,
                                             __bf16* tile, int w, int lane) {
  constexpr int CPR = D / 8, CPS = STRIDE / 8;
#pragma unroll
  for (int m = 0; m < tile_instr_per_wave<STRIDE, NW>(); ++m) {
    const int k = w + NW * m;
    const int q = 64 * k + lane;
    const int r = min(q / CPS, 63), col = min(q % CPS, CPR - 1);
    const __bf16* src = gbase + (long long)min(r, valid - 1) * gst + col * 8;
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(tile + k * 512),
                                     16, 0, 0);
  }
}

// The same copy for a stream of full 64-row tiles with one row stride: the per-lane byte
// offsets inside a tile are computed once (stream_offsets), so each load of a full tile is a
// uniform base plus a VGPR offset (stream_issue). Used with 4-wave workgroups; with fewer
// waves the offsets would cost too many VGPRs and the plain copy is used.
template <int D, int STRIDE, int NW, int M>
__device__ __forceinline__ void stream_offsets(unsigned* off, long long gst, int w, int lane) {
  constexpr int CPR = D / 8, CPS = STRIDE / 8;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int q = 64 * (w + NW * m) + lane;
    const int r = min(q / CPS, 63), col = min(q % CPS, CPR - 1);
    off[m] = (unsigned)((r * gst + col * 8) * 2);
  }
}

template <int D, int STRIDE, int NW, int M>
__device__ __forceinline__ void stream_issue(const unsigned* off, const __bf16* gbase,
                                             long long gst, int valid, __bf16* tile, int w,
                                             int lane) {
  if (valid < 64) {
    wg_copy_tile<D, STRIDE, NW>(gbase, gst, valid, tile, w, lane);
    return;
  }
  const char* b = reinterpret_cast<const char*>(gbase);
#pragma unroll
  for (int m = 0; m < M; ++m)
    __builtin_amdgcn_global_load_lds(b + off[m],
                                     (__attribute__((address_space(3))) void*)(tile + (w + NW * m) * 512),
                                     16, 0, 0);
}

// Wait for this wave's outstanding global loads (including those writing LDS directly).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 16-byte operand: chunk (2 * kstep + half) of row r.
template <int D>
__device__ __forceinline__ bf16x8 lds_frag(const __bf16* tile, int r, int c) {
  return *reinterpret_cast<const bf16x8*>(tile + elem_off<D>(r, c));
}

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;

// A operand of O^T += V^T P^T for M-block md and key k-step ks2, read from V in natural
// [key][d] layout with two transposing reads. In each 16-lane group, lane j points at key
// kseq(j / 4) and the 4 dims 4 * (j % 4) of the group's 16-dim slice; the hardware then hands
// lane i the dim (slice + i) at keys kseq(0..3). Lane l ends up with d = md*32 + l%32 and keys
// 16*ks2 + 4h + {0..3} and 16*ks2 + 8 + 4h + {0..3} (h = l/32): the order in which the S^T
// accumulator, and so P^T, holds them.
template <int D>
__device__ __forceinline__ bf16x8 v_frag(const __bf16* sv, int md, int ks2, int lane) {
  const int grp = lane >> 4, j = lane & 15, hh = lane >> 5;
  const int d = md * 32 + (grp & 1) * 16 + 4 * (j & 3);
  const int key0 = 16 * ks2 + 4 * hh + (j >> 2);
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const int o0 = key0 * Tile<D>::STRV + d;
  const int o1 = o0 + 8 * Tile<D>::STRV;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(sv + o0));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(sv + o1));
  bf16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// S^T[key][row] for one 64-key tile and the wave's 64 rows: s[mb][nb] holds keys
// mb*32 + 8*(v/4) + 4*(lane/32) + v%4 and row nb*32 + lane%32 in element v. Both operands come
// from LDS: K (A operand) from the shared tile, Q^T (B operand) from the wave's own Q rows.
// The four fragments of k-step ks+1 are read while the four MFMAs of step ks run; the
// scheduling fences keep those reads from sinking back next to their use.
template <int D>
__device__ __forceinline__ void qk_tile(const __bf16* sk, const __bf16* sq, f32x16 (&s)[2][2],
                                        int lane) {
  const int rl = lane & 31, hh = lane >> 5;
  bf16x8 qb[2][2], ka[2][2];
  auto load = [&](int ks, int buf) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      qb[buf][n] = lds_frag<D>(sq, n * 32 + rl, 2 * ks + hh);
      ka[buf][n] = lds_frag<D>(sk, n * 32 + rl, 2 * ks + hh);
    }
  };
  load(0, 0);
#pragma unroll
  for (int ks = 0; ks < Tile<D>::KS; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < Tile<D>::KS) load(ks + 1, buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        if (ks == 0) {
          f32x16 z;
#pragma unroll
          for (int v = 0; v < 16; ++v) z[v] = 0.f;
          s[mb][nb] = mfma32(ka[buf][mb], qb[buf][nb], z);
        } else {
          s[mb][nb] = mfma32(ka[buf][mb], qb[buf][nb], s[mb][nb]);
        }
      }
    __builtin_amdgcn_sched_barrier(0);
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
      const bf16x8 a = lds_frag<D>(sk, mb * 32 + rl, 2 * ks + hh);
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
    rmax[nb] = half_max(mx);
  }
}

// Online softmax (BLASST blog, "FlashAttention": running max m, sum l, accumulator O, rescale
// by exp(m_old - m_new)). The exponent reference mref moves only when a row's true max mt
// exceeds it by more than kLazy in the exp2 domain ("rescale ... when needed", paper notes, Key
// Designs 3): exponentials stay <= 2^kLazy and O / l is unchanged, while the O rescale (a VALU
// pass over the accumulators) becomes rare. mt is the exact running max that the relative gate
// compares against.
constexpr float kLazy = 8.f;

struct RowState {
  float mt[2], mref[2], l[2];
};

// Update the running max for a kept tile. Returns true (wave-uniform) when the reference
// moved; alpha then holds the factors O and l must be scaled by after the previous PV.
__device__ __forceinline__ bool softmax_reference(RowState& st, const float (&rmax)[2], float c,
                                                  float (&alpha)[2]) {
  float mn[2];
  bool move = false;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    mn[nb] = fmaxf(st.mt[nb], rmax[nb]);
    st.mt[nb] = mn[nb];
    move |= (mn[nb] - st.mref[nb]) * c > kLazy;    // false for rows that see nothing yet
  }
  const bool moved = __any(move);
  if (moved) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float mu = (mn[nb] == kNegInf) ? 0.f : mn[nb];
      alpha[nb] = __builtin_amdgcn_exp2f((st.mref[nb] - mu) * c);   // 0 on the first block
      st.mref[nb] = mu;
    }
  }
  return moved;
}

// Wait states between VALU writes of P and the first PV MFMA reading it.
__device__ __forceinline__ void pv_operands_ready(bf16x8 (&pb)[2][4]) {
  asm volatile("s_nop 4"
               : "+v"(pb[0][0]), "+v"(pb[0][1]), "+v"(pb[0][2]), "+v"(pb[0][3]),
                 "+v"(pb[1][0]), "+v"(pb[1][1]), "+v"(pb[1][2]), "+v"(pb[1][3]));
}

// Keep P's registers allocated until here (the MFMAs issued before may still read them).
__device__ __forceinline__ void keep_alive(const bf16x8 (&pb)[2][4]) {
  asm volatile("" ::"v"(pb[0][0]), "v"(pb[0][1]), "v"(pb[0][2]), "v"(pb[0][3]), "v"(pb[1][0]),
               "v"(pb[1][1]), "v"(pb[1][2]), "v"(pb[1][3]));
}

// Wait out the MFMA result latency before VALU reads or writes of O (and before the next
// MFMA after a VALU write of O).
template <int MD>
__device__ __forceinline__ void acc_ready(f32x16 (&o)[MD][2]);

template <>
__device__ __forceinline__ void acc_ready<4>(f32x16 (&o)[4][2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[1][0]), "+a"(o[1][1]), "+a"(o[2][0]),
                 "+a"(o[2][1]), "+a"(o[3][0]), "+a"(o[3][1]));
}

template <>
__device__ __forceinline__ void acc_ready<2>(f32x16 (&o)[2][2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[1][0]), "+a"(o[1][1]));
}

// The PV product of the previous kept tile (MFMA, O^T += V^T P^T) interleaved with the
// exponentials of the current kept tile (VALU): each MFMA is issued next to one element pair
// of the softmax, so exp2 / convert / sum run while the matrix core is busy. P is rounded to
// bf16 for the MFMA and l sums exactly those bf16 weights (two per v_dot2 against (1, 1)), so
// O / l stays a convex combination of V rows.
template <int D, bool DO_PV, bool DO_EXP>
__device__ __forceinline__ void pv_exp_block(const __bf16* sv, const bf16x8 (&pbp)[2][4],
                                             f32x16 (&o)[D / 32][2], const f32x16 (&s)[2][2],
                                             const float (&off)[2], float c,
                                             bf16x8 (&pbn)[2][4], float (&sum)[2], int lane) {
  constexpr int MD = D / 32;
  constexpr int NSTEP = MD * 4;               // (k-step, M-block) pairs: 2 MFMAs each
  constexpr int PAIRS = 32;                   // softmax element pairs per lane per tile
  constexpr int PPS = PAIRS / NSTEP;          // pairs per step
  bf16x2 ones;
  ones[0] = (__bf16)1.f;
  ones[1] = (__bf16)1.f;
  bf16x8 pbl[2][4];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2) pbl[nb][ks2] = pbp[nb][ks2];
  bf16x8 vb[3];
  if (DO_PV) {
    pv_operands_ready(pbl);
    vb[0] = v_frag<D>(sv, 0 % MD, 0 / MD, lane);
    vb[1] = v_frag<D>(sv, 1 % MD, 1 / MD, lane);
  }
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {
    const int ks2 = st / MD, md = st % MD;
    if (DO_PV) {
      if (st + 2 < NSTEP) vb[(st + 2) % 3] = v_frag<D>(sv, (st + 2) % MD, (st + 2) / MD, lane);
      mfma_acc(o[md][0], vb[st % 3], pbl[0][ks2]);
      mfma_acc(o[md][1], vb[st % 3], pbl[1][ks2]);
    }
    if (DO_EXP) {
#pragma unroll
      for (int pp = 0; pp < PPS; ++pp) {
        const int pi = st * PPS + pp;
        const int nb = pi / 16, k2 = (pi / 4) % 4, e = 2 * (pi % 4);
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[k2 >> 1][nb][(k2 & 1) * 8 + e], c, off[nb]));
        const float p1 =
            __builtin_amdgcn_exp2f(fmaf(s[k2 >> 1][nb][(k2 & 1) * 8 + e + 1], c, off[nb]));
        bf16x2 pr;
        pr[0] = (__bf16)p0;
        pr[1] = (__bf16)p1;
        sum[nb] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, sum[nb], false);
        pbn[nb][k2][e] = pr[0];
        pbn[nb][k2][e + 1] = pr[1];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (DO_PV) keep_alive(pbl);
}

template <int D>
__device__ __forceinline__ void pv_tile(const __bf16* sv, const bf16x8 (&pb)[2][4],
                                        f32x16 (&o)[D / 32][2], int lane) {
  const f32x16 s0[2][2] = {};
  const float off[2] = {0.f, 0.f};
  bf16x8 dummy[2][4];
  float sum[2] = {0.f, 0.f};
  pv_exp_block<D, true, false>(sv, pb, o, s0, off, 0.f, dummy, sum, lane);
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

// The wave's 64 query rows -> its own LDS tile (swizzled rows; rows past N re-read row N-1,
// their scores are masked).
template <int D>
__device__ __forceinline__ void stage_q(const __bf16* qbase, long long qst, int row0, int N,
                                        __bf16* sq, int lane) {
  wg_copy_tile<D, Tile<D>::STR, 1>(qbase + (long long)row0 * qst, qst, N - row0, sq, 0, lane);
}

template <int D, int BQ, int NW, int GATE>
__global__ __launch_bounds__(NW * 64, 1) void prefill_kernel(PrefillArgs a) {
  constexpr int NT = NW * 64;
  constexpr int WPH = BQ / 64;             // waves per head
  constexpr int HPW = NW / WPH;            // heads per workgroup
  constexpr int MD = Tile<D>::MD;
  constexpr bool kGated = GATE != kDense;

  __shared__ __attribute__((aligned(16))) __bf16 sQ[NW][tile_elems<Tile<D>::STR, 1>()];
  __shared__ __attribute__((aligned(16))) __bf16 sK[2][tile_elems<Tile<D>::STR, NW>()];
  __shared__ __attribute__((aligned(16))) __bf16 sV[2][tile_elems<Tile<D>::STRV, NW>()];
  __shared__ float sGate[2][NW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = tid >> 6;
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
  const float c = a.c_log2;

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

  RowState st;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    st.mt[nb] = kNegInf;
    st.mref[nb] = kNegInf;
    st.l[nb] = 0.f;
  }
  f32x16 o[MD][2];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[md][nb][v] = 0.f;
  acc_ready<MD>(o);

  auto key_valid = [&](int j) { return min(BK, N - j * BK); };
  constexpr int MK = tile_instr_per_wave<Tile<D>::STR, NW>();
  constexpr int MV = tile_instr_per_wave<Tile<D>::STRV, NW>();
  constexpr bool kStream = NW == 4;
  unsigned koff[MK], voff[MV];
  if constexpr (kStream) {
    stream_offsets<D, Tile<D>::STR, NW, MK>(koff, a.ks[1], w, lane);
    stream_offsets<D, Tile<D>::STRV, NW, MV>(voff, a.vs[1], w, lane);
  }
  auto tile_masked = [&](int j) { return j >= n_off || ragged_rows; };

  // Gate statistic of this wave for tile j, in raw score units (the scale is applied at the
  // decision): s_max for ABSOLUTE and DENSE and for the diagonal region in every mode; for
  // RELATIVE off-diagonal tiles, max over the wave's rows of (row max - running max).
  auto publish = [&](int j, const float (&rmax)[2]) {
    float x;
    if (GATE == kRelative && j < n_off) {
      x = kNegInf;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int row = row0 + nb * 32 + (lane & 31);
        x = fmaxf(x, row < N ? rmax[nb] - st.mt[nb] : kNegInf);
      }
    } else {
      x = fmaxf(rmax[0], rmax[1]);
    }
    const float wst = wave_max(x);
    if (lane == 0) sGate[j & 1][w] = wst;
  };

  // ---- prologue: K_0 staged, S_0 computed and published ----
  wg_copy_tile<D, Tile<D>::STR, NW>(Kb, a.ks[1], key_valid(0), sK[0], w, lane);
  wait_vmem();
  __syncthreads();
  if (n_end > 1) wg_copy_tile<D, Tile<D>::STR, NW>(Kb + (long long)BK * a.ks[1], a.ks[1], key_valid(1), sK[1], w, lane);
  f32x16 sc[2][2];   // scores of the tile being processed
  float rc[2];       // their row maxima
  qk_tile<D>(sK[0], sq, sc, lane);
  tile_rowmax(sc, rc, tile_masked(0), 0, row0, N, lane);
  if (want_stat) publish(0, rc);
  wait_vmem();
  __syncthreads();

  int kept = 0;
  bool keep_prev = false;
  bool pending = false;
  float pend[2] = {1.f, 1.f};
  bf16x8 pbp[2][4];   // P of the previous kept tile, consumed by its PV in this iteration

  for (int t = 0; t < n_end; ++t) {
    const int par = t & 1;
    // ---- decision for tile t (statistics visible since the last barrier) ----
    const bool diag = t >= n_off;
    bool mykeep = true, anyv = true;
    if (want_stat) {
      float hst[HPW];
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        float x = sGate[par][hh * WPH];
#pragma unroll
        for (int r = 1; r < WPH; ++r) x = fmaxf(x, sGate[par][hh * WPH + r]);
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

    // V_t (only if some head of the workgroup keeps tile t) and K_{t+2} go straight from
    // global memory into LDS; they are waited for at the end of the iteration
    if constexpr (kStream) {
      if (anyv)
        stream_issue<D, Tile<D>::STRV, NW, MV>(voff, Vb + (long long)t * BK * a.vs[1], a.vs[1],
                                               key_valid(t), sV[par], w, lane);
      if (t + 2 < n_end)
        stream_issue<D, Tile<D>::STR, NW, MK>(koff, Kb + (long long)(t + 2) * BK * a.ks[1],
                                              a.ks[1], key_valid(t + 2), sK[par], w, lane);
    } else {
      if (anyv)
        wg_copy_tile<D, Tile<D>::STRV, NW>(Vb + (long long)t * BK * a.vs[1], a.vs[1],
                                           key_valid(t), sV[par], w, lane);
      if (t + 2 < n_end)
        wg_copy_tile<D, Tile<D>::STR, NW>(Kb + (long long)(t + 2) * BK * a.ks[1], a.ks[1],
                                          key_valid(t + 2), sK[par], w, lane);
    }

    // a reference move of the last kept tile rescales O here: after that tile's predecessor
    // was accumulated (previous iteration) and before its own PV (this iteration)
    if (pending) {
      acc_ready<MD>(o);
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[md][nb][v] *= pend[nb];
      acc_ready<MD>(o);
      pending = false;
    }
    // running max and exponent reference of tile t (kept tiles only)
    float alpha[2] = {1.f, 1.f};
    bool moved = false;
    float off[2] = {0.f, 0.f};
    if (mykeep) {
      moved = softmax_reference(st, rc, c, alpha);
      off[0] = -st.mref[0] * c;
      off[1] = -st.mref[1] * c;
    }
    // PV of the previous kept tile with the exponentials of this one interleaved; when this
    // tile is skipped those exponentials are discarded (VALU work under the PV MFMAs)
    bf16x8 pbn[2][4];
    float sum[2] = {0.f, 0.f};
    if (keep_prev)
      pv_exp_block<D, true, true>(sV[1 - par], pbp, o, sc, off, c, pbn, sum, lane);
    else if (mykeep)
      pv_exp_block<D, false, true>(sV[1 - par], pbp, o, sc, off, c, pbn, sum, lane);
    if (mykeep) {
      if (moved) {
        st.l[0] *= alpha[0];
        st.l[1] *= alpha[1];
        pend[0] = alpha[0];
        pend[1] = alpha[1];
        pending = true;
      }
      st.l[0] += sum[0];
      st.l[1] += sum[1];
    }
    // unconditional: after a skipped tile the next PV is skipped, so pbp is then unused
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int ks2 = 0; ks2 < 4; ++ks2) pbp[nb][ks2] = pbn[nb][ks2];

    // scores of the next tile reuse the registers of this one
    if (t + 1 < n_end) {
      qk_tile<D>(sK[1 - par], sq, sc, lane);
      tile_rowmax(sc, rc, tile_masked(t + 1), (t + 1) * BK, row0, N, lane);
      if (want_stat) publish(t + 1, rc);
    }
    wait_vmem();
    __syncthreads();
    keep_prev = mykeep;
  }
  if (pending) {
    acc_ready<MD>(o);
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[md][nb][v] *= pend[nb];
    acc_ready<MD>(o);
  }
  if (keep_prev) pv_tile<D>(sV[(n_end - 1) & 1], pbp, o, lane);
  acc_ready<MD>(o);

  // ---- epilogue: O / l (renormalised over kept + diagonal), kept counts ----
  const int rl = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float inv = 1.f / half_sum(st.l[nb]);
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

  __shared__ __attribute__((aligned(16))) __bf16 sK[2][tile_elems<Tile<D>::STR, NW>()];
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
    wg_copy_tile<D, Tile<D>::STR, NW>(Kb, a.ks[1], BK, sK[0], w, lane);
    wait_vmem();
    __syncthreads();
    for (int t = 0; t < n_off; ++t) {
      if (t + 1 < n_off)
        wg_copy_tile<D, Tile<D>::STR, NW>(Kb + (long long)(t + 1) * BK * a.ks[1], a.ks[1], BK, sK[(t + 1) & 1],
                            w, lane);
      f32x16 s[2][2];
      float rmax[2];
      qk_tile_regs<D>(sK[t & 1], qf, s, lane);
      tile_rowmax(s, rmax, ragged_rows, t * BK, row0, N, lane);
      const float st = wave_max(fmaxf(rmax[0], rmax[1]));
      if (lane == 0) sW[w][t] = st * a.scale;
      wait_vmem();
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
