// Device code of the exact-score-gated block-sparse causal prefill attention for gfx950 (MI355X).
// Included by the translation units that instantiate the kernels (one per head dimension,
// query tile and K/V layout, so that they compile in parallel).
//
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
//   * One wavefront owns 32 query rows of one head, and two wavefronts share each SIMD, so the
//     exponentials of one issue on the vector ALU while the other's matrix instructions run.
//     Scores are produced transposed, S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K from
//     LDS, B = Q^T resident in VGPRs): each lane holds 32 scores of its row, so the row max is
//     an in-lane max chain plus one exchange between the two half-waves, and the exponentials
//     stay in the lanes that produced them.
//   * O^T = V^T P^T: P^T is the MFMA B operand straight from the softmax registers; V^T is read
//     from the natural [key][d] V tile with transposing LDS reads, in the key order in which
//     the S^T accumulator (and so P^T) holds them.
//   * A workgroup holds the 32-row waves of the query rows of one query block that share a KV
//     head: one head x 128 rows (4 waves) for the 128x64 tile, two heads x 64 rows for the
//     64x64 tile. Each K/V tile is staged in LDS once per workgroup, by direct global->LDS
//     loads, and read by every wave; K and V are double-buffered. (A whole KV group of four
//     heads x 128 rows does not fit one CU at two waves per SIMD: 16 waves of ~230 VGPRs, or Q
//     of 128 KB in LDS beside the K/V buffers. The gate sweep, which holds no softmax state,
//     takes two heads per workgroup; its FP8 form four.)
//   * QK of tile t+1 is issued after the softmax of tile t, so the gate statistics of tile t+1
//     reach LDS before the one barrier of the iteration; V_t is fetched only when some head of
//     the workgroup keeps tile t.
//   * Workgroups are ordered heaviest query block first, and (when the unit count allows)
//     all query blocks of one KV head go to the same XCD so their K/V stream shares its L2.
#pragma once

#include "bsfa_internal.h"

#include <math.h>

#include <type_traits>

namespace bsfa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((address_space(3))) void lds_void;

template <int V>
using IC = std::integral_constant<int, V>;

// Calls f(IC<i>{}) for i = I .. E-1 (compile-time loop index).
template <int I, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(IC<I>{});
    static_for<I + 1, E>(f);
  }
}

constexpr int BK = kBlockK;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bits_f(int x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ int f_bits(float x) { return __builtin_bit_cast(int, x); }

// max(a, b, c) as one v_max3_f32 without the operand canonicalisation that fmaxf implies in
// IEEE mode (scores are finite or -inf here, never NaN). The compiler cannot see into the asm,
// so it cannot insert the wait states the hardware needs between an MFMA writing a VGPR and a
// vector instruction reading it: a block of MFMA results is first read by a compiler-visible
// instruction (first_max(), which the compiler delays as far as the hazard requires), and the
// asm reads of the block follow it in the dependency chain.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float first_max(float acc, float a, float b) {
  return fmaxf(acc, fmaxf(a, b));
}
// max3 that is ordered after `dep` (an unused input), for asm reads of a block of MFMA results
// that do not otherwise depend on its compiler-visible first read.
__device__ __forceinline__ float max3_after(float a, float b, float c, float dep) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c), "v"(dep));
  return r;
}

// max over the 16 scores of one MFMA result block and acc, as a shallow tree (the reduction
// ends the iteration's critical path).
__device__ __forceinline__ float block_max(float acc, const f32x16& s) {
  const float a = first_max(acc, s[0], s[1]);
  const float m1 = max3_after(s[2], s[3], s[4], a);
  const float m2 = max3_after(s[5], s[6], s[7], a);
  const float m3 = max3_after(s[8], s[9], s[10], a);
  const float m4 = max3_after(s[11], s[12], s[13], a);
  const float m5 = max3_after(s[14], s[15], s[15], a);
  return max3(max3(a, m1, m2), max3(m3, m4, m5), m5);
}

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

// Wave-uniform sum over the 64 lanes, the butterfly of wave_max with additions.
__device__ __forceinline__ int wave_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xf, 0xf, false);    // quad_perm [1,0,3,2]
  x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xf, 0xf, false);    // quad_perm [2,3,0,1]
  x += __builtin_amdgcn_update_dpp(0, x, 0x141, 0xf, 0xf, false);   // row_half_mirror
  x += __builtin_amdgcn_update_dpp(0, x, 0x140, 0xf, 0xf, false);   // row_mirror
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) +
         __builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48);
}

// Wait for this wave's outstanding global loads (including those writing LDS directly).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wave's global loads are outstanding (they complete in order).
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt field");   // bits 3:0 and 15:14
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

template <int D>
struct Tile {
  static constexpr int CPR = D / 8;         // 16-byte chunks of data per row (16 or 8)
  static constexpr int STR = D + 8;         // K row stride in bf16 (one 16-byte pad chunk)
  static constexpr int STRV = D + 32;       // V row stride in bf16 (four pad chunks)
  static constexpr int KS = D / 16;         // QK k-steps over d
  static constexpr int MD = D / 32;         // PV M-blocks over d
};

// LDS tiles hold 64 rows of D bf16 plus padding, so that every fragment address is a per-lane
// base plus a compile-time offset, and the rows one read touches spread over the 64 banks:
//   * K (row stride D + 8): a 16-byte operand read covers 16 consecutive rows per 16 lanes;
//     rows start 4 banks apart, so the 16 reads tile all 64 banks.
//   * V (row stride D + 32): a transposing read covers 4 consecutive rows x 64 bytes per 32
//     lanes; rows start 16 banks apart, so the 4 row segments are disjoint.
//
// Tiles are filled by direct global -> LDS loads, 1 KB per instruction: lane l of instruction k
// fills padded chunk q = 64k + l (row q / CPS, column q % CPS, CPS = STRIDE / 8 chunks per
// padded row) with the matching global chunk; pad chunks re-fetch the row's last chunk. A tile
// is exactly CPS instructions. Rows at or past `valid` re-read row valid - 1 (their scores are
// masked and their P weights are zero).

// ---------------------------------------------------------------------------------------------
// Workgroup-wide tile copies. Wave w of NW issues instructions k = w + NW*m.
// ---------------------------------------------------------------------------------------------
template <int STRIDE, int NW>
constexpr int copy_iters() {
  return (STRIDE / 8 + NW - 1) / NW;
}

// Per-lane byte offsets, inside a full tile, of the chunks this wave copies (computed once per
// workgroup; 32-bit because the host bounds the token stride so that 64 rows stay below 4 GB).
template <int D, int STRIDE, int NW>
__device__ __forceinline__ void copy_offsets(unsigned* off, long long gst, int w, int lane) {
  constexpr int CPR = D / 8, CPS = STRIDE / 8, M = copy_iters<STRIDE, NW>();
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int q = 64 * min(w + NW * m, CPS - 1) + lane;
    const int r = q / CPS, col = min(q % CPS, CPR - 1);
    off[m] = (unsigned)(r * (unsigned)gst + col * 8) * 2u;
  }
}

// 32-bit LDS byte address of a __shared__ object (the cast checks for null, so it is done once
// per buffer, outside the loops; the copies take these addresses, never generic pointers).
__device__ __forceinline__ unsigned lds_addr(const void* lds) {
  typedef __attribute__((address_space(3))) const char lds_char;
  return __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_char*)lds);
}

// One direct global -> LDS copy instruction (16 bytes per lane, lane l to LDS byte address
// lds + 16 l), issued through inline asm: the compiler then does not track it, and in
// particular does not make later LDS reads (of other buffers) wait for it; whoever reads the
// destination waits for it with wait_vmem() before a barrier. gbase and lds are wave-uniform,
// voff per lane. M0 (the LDS destination) is saved and restored around the copy. The scalar
// operands may have just been written by v_readfirstlane, and a memory instruction reading an
// SGPR written by a vector instruction needs 5 wait states; the asm supplies them itself (the
// compiler cannot see the read): two moves plus s_nop 2.
__device__ __forceinline__ void dma16_at(const void* gbase, unsigned voff, unsigned lds) {
  const unsigned long long g = reinterpret_cast<unsigned long long>(gbase);
  const unsigned glo = __builtin_amdgcn_readfirstlane((unsigned)g);
  const unsigned ghi = __builtin_amdgcn_readfirstlane((unsigned)(g >> 32));
  const unsigned long long gs = ((unsigned long long)ghi << 32) | glo;
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 2\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(gs), "s"(m0)
      : "memory");
}

// Round m of a tile copy into the LDS buffer at byte address lds: instruction k = w + NW*m
// of the tile, if it exists (wave-uniform; only the last round can run past the tile). For a
// ragged tile (valid < 64 rows) the chunks of rows at or past `valid` are redirected to row
// valid - 1.
template <int D, int STRIDE, int NW>
__device__ __forceinline__ void copy_round(int m, const unsigned* off, const __bf16* gbase,
                                           unsigned row_bytes, int valid, unsigned lds, int w,
                                           int lane) {
  constexpr int CPS = STRIDE / 8, M = copy_iters<STRIDE, NW>();
  const int k = w + NW * m;
  if (m + 1 < M || k < CPS) {
    unsigned o = off[m];
    if (valid < 64) {
      const int r = (64 * k + lane) / CPS;
      o -= (unsigned)max(r - (valid - 1), 0) * row_bytes;
    }
    dma16_at(gbase, o, lds + k * 1024u);
  }
}

// Round m of the copy of a whole 64-row tile (valid = 64) into the LDS buffer at byte address
// lds: no ragged-row handling, the destination a precomputed LDS address (the steady state of
// the softmax loop; a ragged tile goes through copy_round).
template <int D, int STRIDE, int NW>
__device__ __forceinline__ void copy_round_full(int m, const unsigned* off, const __bf16* gbase,
                                                unsigned lds, int w) {
  constexpr int CPS = STRIDE / 8, M = copy_iters<STRIDE, NW>();
  const int k = w + NW * m;
  if (m + 1 < M || k < CPS) dma16_at(gbase, off[m], lds + k * 1024u);
}

// Copy one 64-row tile starting at gbase (all rounds) into the LDS buffer at byte address lds.
template <int D, int STRIDE, int NW>
__device__ __forceinline__ void copy_tile(const unsigned* off, const __bf16* gbase,
                                          unsigned row_bytes, int valid, unsigned lds, int w,
                                          int lane) {
#pragma unroll
  for (int m = 0; m < copy_iters<STRIDE, NW>(); ++m)
    copy_round<D, STRIDE, NW>(m, off, gbase, row_bytes, valid, lds, w, lane);
}

// ---------------------------------------------------------------------------------------------
// Operand fragments
// ---------------------------------------------------------------------------------------------

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

// B operand Q^T of S^T = K Q^T for 32 query rows: lane l holds row row0 + l%32 and dims
// 16*ks + 8*(l/32) + {0..7} in qf[ks]. Rows past N are zero.
template <int D>
__device__ __forceinline__ void load_q32(const __bf16* qbase, long long qst, int row0, int N,
                                         bf16x8 (&qf)[D / 16], int lane) {
  const int row = row0 + (lane & 31);
  const __bf16* p = qbase + (long long)min(row, N - 1) * qst + 8 * (lane >> 5);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const uint4 x = *reinterpret_cast<const uint4*>(p + 16 * ks);
    qf[ks] = __builtin_bit_cast(bf16x8, row < N ? x : make_uint4(0, 0, 0, 0));
  }
}

// S^T[key][row] for one 64-key tile and the wave's 32 rows: s[mb] holds keys
// mb*32 + 8*(v/4) + 4*(lane/32) + v%4 of row lane%32 in element v. The two K fragments of
// k-step ks+1 are read while the two MFMAs of step ks run.
template <int D>
__device__ __forceinline__ void qk32(const __bf16* sk, const bf16x8 (&qf)[D / 16],
                                     f32x16 (&s)[2], int lane) {
  constexpr int KS = Tile<D>::KS, STR = Tile<D>::STR;
  const __bf16* base = sk + (lane & 31) * STR + 8 * (lane >> 5);
  bf16x8 ka[2][2];
  auto load = [&](int ks, int buf) {
    ka[buf][0] = *reinterpret_cast<const bf16x8*>(base + 16 * ks);
    ka[buf][1] = *reinterpret_cast<const bf16x8*>(base + 32 * STR + 16 * ks);
  };
  load(0, 0);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < KS) load(ks + 1, buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    if (ks == 0) {
      f32x16 z;
#pragma unroll
      for (int v = 0; v < 16; ++v) z[v] = 0.f;
      s[0] = mfma32(ka[buf][0], qf[ks], z);
      s[1] = mfma32(ka[buf][1], qf[ks], z);
    } else {
      s[0] = mfma32(ka[buf][0], qf[ks], s[0]);
      s[1] = mfma32(ka[buf][1], qf[ks], s[1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Causal / ragged masking (when `masked`) and the row max over the 64 keys of the tile.
// arow: the lane's query row as an absolute position (the causal compare); rvalid: the row
// exists (rows past the end of a ragged last block do not).
__device__ __forceinline__ float rowmax32(f32x16 (&s)[2], bool masked, int key0, int arow,
                                          bool rvalid, int lane) {
  const int hh = lane >> 5;
  if (masked) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = key0 + mb * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (key > arow || !rvalid) s[mb][v] = kNegInf;
      }
  }
  float mx = kNegInf;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int v = 0; v < 16; v += 2)
      mx = (v == 0) ? first_max(mx, s[mb][v], s[mb][v + 1]) : max3(mx, s[mb][v], s[mb][v + 1]);
  return half_max(mx);
}

// Online softmax (BLASST blog, "FlashAttention": running max m, sum l, accumulator O, rescale
// by exp(m_old - m_new)). The exponent reference mref moves only when a row's true max mt
// exceeds it by more than kLazy in the exp2 domain: exponentials stay <= 2^kLazy and O / l is
// unchanged, while the O rescale (a vector pass over the accumulators) becomes rare. mt is the
// exact running max that the relative gate compares against.
constexpr float kLazy = 8.f;

struct RowState {
  float mt, mref, l;
};

// Update the running max for a kept tile. Returns true (wave-uniform) when the reference
// moved; alpha then holds the factor O and l must be scaled by after the previous PV.
__device__ __forceinline__ bool update_reference(RowState& st, float rmax, float c,
                                                 float& alpha) {
  const float mn = fmaxf(st.mt, rmax);
  st.mt = mn;
  const bool moved = __any((mn - st.mref) * c > kLazy);   // false for rows that see nothing yet
  if (moved) {
    const float mu = (mn == kNegInf) ? 0.f : mn;
    alpha = __builtin_amdgcn_exp2f((st.mref - mu) * c);   // 0 on the first block
    st.mref = mu;
  }
  return moved;
}

// One pair of P entries of the current tile: exponentials of the scaled scores against the
// exponent reference (off = -mref * c), rounded to bf16 for the PV MFMA, and their sum added to
// the row sum; l sums exactly the bf16 weights the MFMA uses (two per v_dot2 against (1, 1)),
// so O / l stays a convex combination of V rows. Pair p covers P^T elements 2(p%4), 2(p%4)+1
// of k-step p/4, i.e. scores s[p/8][8 ((p/4) % 2) + 2(p%4) + {0, 1}].
__device__ __forceinline__ void exp_pair(int p, const f32x16 (&s)[2], float off, float c,
                                         bf16x8 (&pbn)[4], float& sum) {
  const int k2 = p / 4, e = 2 * (p % 4);
  const float p0 = __builtin_amdgcn_exp2f(fmaf(s[k2 >> 1][(k2 & 1) * 8 + e], c, off));
  const float p1 = __builtin_amdgcn_exp2f(fmaf(s[k2 >> 1][(k2 & 1) * 8 + e + 1], c, off));
  bf16x2 pr, ones;
  pr[0] = (__bf16)p0;
  pr[1] = (__bf16)p1;
  ones[0] = (__bf16)1.f;
  ones[1] = (__bf16)1.f;
  sum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, sum, false);
  pbn[k2][e] = pr[0];
  pbn[k2][e + 1] = pr[1];
}

constexpr int kPairs = 16;        // P pairs per lane per tile (32 rows x 64 keys / 64 lanes / 2)
// Of these, the dense and mask-walk loops issue the first kPairsPV next to the PV MFMAs and the
// rest next to the QK MFMAs; the voting kernels issue all of them next to the QK MFMAs.
constexpr int kPairsPV = 8;

// Steps [FIRST, LAST) of the PV product of the previous kept tile (O^T += V^T P^T, one MFMA per
// (k-step, M-block); fragments read two steps ahead into vb, the first two by pv_prefetch)
// with, next to the MFMAs, exponential pairs 0 .. NPV-1 of the current tile (do_exp) and
// the MV rounds of the V_t copy (vload, copy_v(r)), both spread over steps DEC .. NSTEP-1.
template <int D>
__device__ __forceinline__ void pv_prefetch(const __bf16* sv, bf16x8 (&vb)[3], int lane) {
  constexpr int MD = D / 32;
  vb[0] = v_frag<D>(sv, 0, 0, lane);
  vb[1] = v_frag<D>(sv, 1 % MD, 1 / MD, lane);
}

// How a step sequence treats each of its optional parts: kNever (compiled out), kFlag (a
// wave-uniform run-time flag tested at every step) or kAlways (straight-line code). Per-step
// tests cost a compare and a branch each; the common cases are compiled without them.
enum PartMode : int { kNever = 0, kFlag = 1, kAlways = 2 };
__device__ __forceinline__ bool part_on(int mode, bool flag) {
  return mode == kAlways || (mode == kFlag && flag);
}

template <int D, int FIRST, int LAST, int DEC, int MV, int PVM = kFlag, int EXM = kFlag,
          int VLM = kFlag, int NPV = kPairsPV, typename CopyV>
__device__ __forceinline__ void pv_steps(bool do_pv, bool do_exp, bool vload, const __bf16* sv,
                                         const bf16x8 (&pbp)[4], f32x16 (&o)[D / 32],
                                         bf16x8 (&vb)[3], const f32x16 (&sc)[2], float off,
                                         float c, bf16x8 (&pbn)[4], float& sum, int lane,
                                         CopyV&& copy_v) {
  do_pv = part_on(PVM, do_pv);
  do_exp = part_on(EXM, do_exp);
  vload = part_on(VLM, vload);
  constexpr int MD = D / 32;
  constexpr int NSTEP = MD * 4;
  constexpr int NE = NSTEP - DEC > 0 ? NSTEP - DEC : 1;
  static_for<FIRST, LAST>([&](auto stc) {
    constexpr int st = decltype(stc)::value;
    constexpr int ks2 = st / MD, md = st % MD;
    if (do_pv) {
      if constexpr (st + 2 < NSTEP)
        vb[(st + 2) % 3] = v_frag<D>(sv, (st + 2) % MD, (st + 2) / MD, lane);
      o[md] = mfma32(vb[st % 3], pbp[ks2], o[md]);
    }
    if (vload) {
#pragma unroll
      for (int r = 0; r < MV; ++r)
        if (DEC + r * NE / MV == st) copy_v(r);
    }
    if (do_exp && st >= DEC) {
#pragma unroll
      for (int pi = (st - DEC) * NPV / NE; pi < (st - DEC + 1) * NPV / NE; ++pi)
        exp_pair(pi, sc, off, c, pbn, sum);
    }
    __builtin_amdgcn_sched_barrier(0);
  });
}

// S^T = K Q^T for the next tile, M-block outer (step st: block st / KS, k-step st % KS), each
// step reading the next step's K fragment. Next to the MFMAs: the MK rounds of the K_{t+2}
// copy (kload, copy_k(r)) on the first steps and the MV rounds of a V copy (vload, copy_v(r))
// on the last ones, the remaining exponential pairs of the current tile (do_exp) and, during
// the second M-block, the in-lane max over the first block's 16 scores (into mx).
template <int D, int MK, int EXM = kFlag, int KLM = kFlag, int NPV = kPairsPV, int MV = 1,
          int VLM = kNever, typename CopyK, typename CopyV>
__device__ __forceinline__ void qk_phase(bool do_exp, bool kload, const __bf16* kbase,
                                         const bf16x8 (&qf)[D / 16],
                                         f32x16 (&sn)[2], const f32x16 (&sc)[2], float off,
                                         float c, bf16x8 (&pbn)[4], float& sum, float& mx,
                                         CopyK&& copy_k, bool vload, CopyV&& copy_v) {
  do_exp = part_on(EXM, do_exp);
  kload = part_on(KLM, kload);
  vload = part_on(VLM, vload);
  constexpr int KS = Tile<D>::KS, STR = Tile<D>::STR, NST = 2 * KS;
  constexpr int NP = kPairs - NPV;
  bf16x8 ka[2];
  ka[0] = *reinterpret_cast<const bf16x8*>(kbase);
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    const int mb = st / KS, ks = st % KS;
    const int buf = st & 1;
    if (st + 1 < NST) {
      const int mb1 = (st + 1) / KS, ks1 = (st + 1) % KS;
      ka[buf ^ 1] = *reinterpret_cast<const bf16x8*>(kbase + mb1 * 32 * STR + 16 * ks1);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (ks == 0) {
      f32x16 z;
#pragma unroll
      for (int v = 0; v < 16; ++v) z[v] = 0.f;
      sn[mb] = mfma32(ka[buf], qf[0], z);
    } else {
      sn[mb] = mfma32(ka[buf], qf[ks], sn[mb]);
    }
    if (kload) {
#pragma unroll
      for (int r = 0; r < MK; ++r)
        if (r * (NST / 2) / MK == st) copy_k(r);
    }
    if (vload) {
#pragma unroll
      for (int r = 0; r < MV; ++r)
        if (NST / 2 + r * (NST / 2) / MV == st) copy_v(r);
    }
    if (do_exp) {
#pragma unroll
      for (int pi = NPV + st * NP / NST; pi < NPV + (st + 1) * NP / NST; ++pi)
        exp_pair(pi, sc, off, c, pbn, sum);
    }
    if (mb == 1) {
#pragma unroll
      for (int e = ks * 16 / KS; e < (ks + 1) * 16 / KS; e += 2)
        mx = e == 0 ? first_max(mx, sn[0][e], sn[0][e + 1]) : max3(mx, sn[0][e], sn[0][e + 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Causal / ragged mask of a score tile (diagonal-region and ragged tiles only); arow and rvalid
// as for rowmax32.
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int key0, int arow, bool rvalid,
                                          int lane) {
  const int hh = lane >> 5;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = key0 + mb * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
      if (key > arow || !rvalid) s[mb][v] = kNegInf;
    }
}

struct Unit {
  int b, g, hg, i;
};

// The sequence a workgroup works on: its query rows N, key tokens Nk, the prefix pre = Nk - N
// (query row r sits at absolute position pre + r) and the element offsets of its first token in
// Q, K, V and O. A fixed-length batch strides by the batch axis; a variable-length batch packs
// its sequences along the token axis, with their token offsets in cu_q / cu_k.
struct Seq {
  int N, Nk, pre;
  long long q, k, v, o;
};

__device__ __forceinline__ Seq seq_of(const PrefillArgs& a, int b) {
  Seq s;
  if (a.cu_q) {
    const int q0 = a.cu_q[b];
    s.N = a.cu_q[b + 1] - q0;
    s.q = (long long)q0 * a.qs[1];
    s.o = (long long)q0 * a.os[1];
    if (a.pages) {   // paged keys: tile addresses come from the page table (tile_offset)
      s.Nk = a.kv_lens[b];
      s.k = s.v = 0;
    } else {
      const int k0 = a.cu_k[b];
      s.Nk = a.cu_k[b + 1] - k0;
      s.k = (long long)k0 * a.ks[1];
      s.v = (long long)k0 * a.vs[1];
    }
  } else {
    s.N = a.N;
    s.Nk = a.Nk;
    s.q = b * a.qs[0];
    s.o = b * a.os[0];
    s.k = b * a.ks[0];
    s.v = b * a.vs[0];
  }
  s.pre = s.Nk - s.N;
  return s;
}

// Workgroup L -> (batch, KV head, head group, query block). Query blocks go from the last
// (longest) to the first. Consecutive workgroups land on the 8 XCDs in turn (L mod 8); with
// xcd_map the unit index is chosen so that XCD x serves fixed units (for B * Hkv = 8: KV head
// x), which keeps each XCD's L2 on one K/V stream when the workgroups sweep it in step. A
// nonzero xcd_rot turns that assignment by one every xcd_rot query blocks (about the number
// in flight at once), so that over the launch every XCD serves every KV head equally often:
// for walks whose length differs between heads, the XCDs then finish together.
__device__ __forceinline__ Unit decode_unit(int L, int units, int nqb, int B, int Hkv,
                                            int xcd_map, int xcd_rot, int tail = 0) {
  int i, u;
  if (xcd_map < 0 && L < (nqb - tail) * units) {
    // KV-head-major: every (batch, KV head) in turn, its query blocks from the last, its head
    // groups innermost. Consecutive workgroups still go to the 8 XCDs in turn, so all XCDs
    // work on the same KV head at a time and its K/V (64 MB at 128K, d = 128) stays in the
    // last-level cache for every XCD's walk. Only the query blocks at or above `tail` are
    // taken in this order; the rest follow below.
    const int upg = units / (B * Hkv), nb = nqb - tail;
    const int bh = L / (nb * upg), rem = L % (nb * upg);
    Unit r;
    r.b = bh / Hkv;
    r.g = bh % Hkv;
    r.i = nqb - 1 - rem / upg;
    r.hg = rem % upg;
    return r;
  }
  if (xcd_map < 0) {
    // The query blocks below `tail`, last, heaviest first, each with the units of every KV
    // head: the launch ends on the shortest units whatever the KV head order, so no workgroup
    // is left with a long unit of the last KV head while the others have run out of work.
    L -= (nqb - tail) * units;
    i = tail - 1 - L / units;
    u = L % units;
  } else if (xcd_map) {
    const int x = L & 7, s = L >> 3, upx = units >> 3;
    i = nqb - 1 - s / upx;
    u = (s % upx) * 8 + (xcd_rot ? ((x + (nqb - 1 - i) / xcd_rot) & 7) : x);
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

// Element offset (from the sequence's base) of 64-key tile j in K or V (token stride tst, page
// stride pst). Contiguous sequences stride by tiles; a paged cache looks the tile's page up in
// the block table: pages hold a whole number of tiles, so a tile never straddles two.
template <bool PAGED>
__device__ __forceinline__ long long tile_offset(const PrefillArgs& a, int b, int j,
                                                 long long tst, long long pst) {
  if constexpr (PAGED) {
    const int page = a.pages[(long long)b * a.pages_stride + j / a.page_tiles];
    return (long long)page * pst + (long long)(j % a.page_tiles) * kBlockK * tst;
  }
  return (long long)j * kBlockK * tst;
}

// ---------------------------------------------------------------------------------------------
// Prefill kernel
// ---------------------------------------------------------------------------------------------
constexpr int kRows = kRowsPerWave;

constexpr int kMaskWords = kMaxGateTiles / 64;   // keep-bitmask words

// How a prefill launch hands out its units: the mask walk always takes them from a ticket
// counter; dense, and the voting gates with one head per workgroup, do when the call brings
// a counter (a workspace), else run one workgroup per unit. (The unit loop holds a few more
// registers across units: the relative gate's two-head form would spill.)
enum UnitLoop : int { kOnePerUnit, kTicketIfGiven, kTicketAlways };
template <int GATE, int HPW>
constexpr int kUnitLoop = GATE == kAbsolute ? kTicketAlways
                          : GATE == kDense || HPW == 1 ? kTicketIfGiven : kOnePerUnit;

// PAGED: K and V tiles come from a paged cache (a compile-time choice, so that the contiguous
// kernels carry no page lookups). MEAN (absolute walk only): the pruned gate blocks' stand-ins
// join the softmax after the walk (mean correction).
template <int D, int BQ, int NW, int GATE, bool PAGED, bool MEAN = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(
    PrefillArgs a) {
  constexpr int WPH = BQ / kRows;          // waves per head
  constexpr int HPW = NW / WPH;            // heads per workgroup
  constexpr int MD = Tile<D>::MD, KS = Tile<D>::KS;
  constexpr int STR = Tile<D>::STR, STRV = Tile<D>::STRV;
  constexpr int MK = copy_iters<STR, NW>(), MV = copy_iters<STRV, NW>();
  // ABSOLUTE: the gate of a block depends only on its own maximum, so all off-diagonal
  // maxima are found first (pass 1, scores only) and the softmax then runs over the kept
  // tiles and the diagonal region (pass 2). RELATIVE decides tile by tile inside the loop.
  constexpr bool kAbs = GATE == kAbsolute;          // walks the gate sweep's keep masks
  constexpr bool kThr = kAbs || GATE == kAbsVote;    // thresholds from the table
  static_assert(!kThr || HPW == 1, "the absolute gate runs one head per workgroup");
  static_assert(!MEAN || kAbs, "mean correction walks the gate sweep's masks");

  // Separate objects per buffer: the compiler then sees that a direct copy into one buffer
  // cannot alias reads of the other and does not wait for the copy before those reads.
  __shared__ __attribute__((aligned(16))) __bf16 sK0[64 * STR];
  __shared__ __attribute__((aligned(16))) __bf16 sK1[64 * STR];
  __shared__ __attribute__((aligned(16))) __bf16 sV0[64 * STRV];
  __shared__ __attribute__((aligned(16))) __bf16 sV1[64 * STRV];
  __shared__ __attribute__((aligned(16))) float sGate[2][NW * kRows];   // per-row gate statistics
  __shared__ unsigned long long sMask[kAbs ? kMaskWords : 1];           // kept off-diagonal tiles
  __shared__ int sKept[kAbs ? NW : 1];   // per-wave kept-tile counts of the mask walk
  __shared__ int sUnit;

  // Workgroup L runs unit L, unless the launch has a ticket counter (zero at the launch): then
  // it holds as many workgroups as stay resident, and each takes units in turn from the
  // counter until none is left. Workgroups go to the XCDs in turn whatever their work, and a
  // new one waits for a slot on its own XCD; as unit lengths vary (a walk's kept tiles, a
  // query block's causal extent), slots would sit idle on the other XCDs meanwhile. Resident
  // workgroups that take the next unit as they finish one keep every slot busy until the work
  // runs out.
  const unsigned lK0 = lds_addr(sK0), lK1 = lds_addr(sK1);
  const unsigned lV0 = lds_addr(sV0), lV1 = lds_addr(sV1);
  constexpr bool kLoop = kUnitLoop<GATE, HPW> != kOnePerUnit;
  const bool tickets = kUnitLoop<GATE, HPW> == kTicketAlways || a.ticket != nullptr;   // uniform
  int L = blockIdx.x;
next_unit:
  if (kLoop && tickets) {
    if (threadIdx.x == 0) sUnit = (int)atomicAdd(a.ticket, 1u);
    __syncthreads();
    L = __builtin_amdgcn_readfirstlane(sUnit);
    if (L >= a.units * a.nqb) return;   // uniform: every unit taken
  }
  // (with mean correction and in the voting gates the lane and wave indices are made opaque
  // per unit: otherwise the compiler computes some lane-dependent offsets once ahead of the
  // unit loop and holds them through it, which spills)
  int tid_u = threadIdx.x, w_u = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  if constexpr (kLoop && (MEAN || GATE == kRelative || GATE == kAbsVote)) {
    asm volatile("" : "+v"(tid_u));
    asm volatile("" : "+s"(w_u));
  }
  const int tid = tid_u, lane = tid & 63;
  const int w = w_u;   // wave index, in a scalar register
  const int hw = w / WPH, rw = w % WPH;
  const Unit un = decode_unit(L, a.units, a.nqb, a.B, a.Hkv, a.xcd_map, a.xcd_rot,
                              a.tail_blocks);
  const int b = un.b, g = un.g, i = un.i;
  const int h0 = g * a.G + un.hg * HPW;
  const int h = h0 + hw;
  // N query rows at absolute positions pre .. pre + N - 1 against Nk = pre + N keys (a chunk
  // after a prefix of cached keys; pre = 0 for a whole prefill)
  const Seq sq = seq_of(a, b);
  if (i * BQ >= sq.N) {          // uniform: past this sequence's query blocks (variable length)
    if (kLoop && tickets) {
      __syncthreads();             // every wave has read sUnit
      goto next_unit;
    }
    return;
  }
  const int N = sq.N, Nk = sq.Nk, pre = sq.pre;
  const int row0 = i * BQ + rw * kRows;
  const int row = row0 + (lane & 31);
  const int arow = pre + row;
  const bool rvalid = row < N;
  const int n_off = (pre + i * BQ) / BK;
  const int n_end = (pre + min((i + 1) * BQ, N) - 1) / BK + 1;
  const bool ragged_rows = (i + 1) * BQ > N;
  const bool head_leader = (rw == 0) && (lane == 0);
  const float c = a.c_log2;

  const __bf16* Qb = static_cast<const __bf16*>(a.q) + sq.q + h * a.qs[2];
  const __bf16* Kb = static_cast<const __bf16*>(a.k) + sq.k + g * a.ks[2];
  const __bf16* Vb = static_cast<const __bf16*>(a.v) + sq.v + g * a.vs[2];
  const long long kst = a.ks[1], vst = a.vs[1];

  float thr[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    if (kThr)   // the absolute query block's column (pre is a multiple of BQ here)
      thr[hh] = a.thr[(h0 + hh) * a.t_len + min(pre / BQ + i, a.t_len - 1)];
    else if (GATE == kRelative)
      thr[hh] = a.log_lambda;
    else
      thr[hh] = kNegInf;
  }
  // How the absolute gate decides: kAbsolute walks only the kept tiles of the gate sweep's
  // keep mask (two_pass); kAbsVote decides each tile in the loop like the relative gate
  // (loop_gate, a vote of the rows on s_max >= T). A threshold of -inf keeps every block, so
  // nothing needs deciding then (unless the maxima are dumped).
  const bool decide = kThr && n_off > 0 && (thr[0] != kNegInf || a.dbg != nullptr);
  const bool two_pass = kAbs && decide;
  const bool loop_gate = GATE == kRelative || (GATE == kAbsVote && decide);
  const bool want_stat = loop_gate || a.dbg != nullptr;

  unsigned koff[MK], voff[MV];
  copy_offsets<D, STR, NW>(koff, kst, w, lane);
  copy_offsets<D, STRV, NW>(voff, vst, w, lane);
  auto key_valid = [&](int j) { return min(BK, Nk - j * BK); };
  const unsigned krow = (unsigned)kst * 2u, vrow = (unsigned)vst * 2u;
  auto load_k = [&](int j, unsigned dst) {
    copy_tile<D, STR, NW>(koff, Kb + tile_offset<PAGED>(a, b, j, kst, a.ks[0]), krow, key_valid(j),
                          dst, w, lane);
  };

  bf16x8 qf[KS];
  load_q32<D>(Qb, a.qs[1], row0, N, qf, lane);
  auto tile_masked = [&](int j) { return j >= n_off || ragged_rows; };

  // ---- the gate sweep's keep mask of this (b, h, i), staged in LDS and counted ----
  int kept = 0, kept_all = 0;
  if (two_pass) {
    const int nw64 = (n_off + 63) >> 6;
    const unsigned long long* gm =
        a.keep_mask + (((long long)b * a.Hq + h) * a.nqb + i) * a.mask_words;
    // each word counted by the thread that stages it; a wave sum, then the waves' sums
    int cnt = 0;
    for (int x = tid; x < nw64; x += NW * 64) {
      const unsigned long long word = gm[x];
      sMask[x] = word;
      cnt += __builtin_popcountll(word);
    }
    cnt = wave_sum(cnt);
    if (lane == 0) sKept[w] = cnt;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NW; ++k) kept_all += sKept[k];
    kept = kept_all / a.kpb;   // kept gate blocks (a kept block sets all its tiles' bits)
  } else if (!loop_gate) {
    // dense, or an absolute threshold of -inf: every off-diagonal gate block kept
    kept = (pre + i * BQ) / (BK * a.kpb);
  }
  // The tile after j in the sequence the softmax walks: with the pass-1 mask, the next kept
  // off-diagonal tile and then the diagonal region; otherwise every tile.
  auto next_tile = [&](int j) -> int {
    ++j;
    if (!two_pass || j >= n_off) return j;
    int wi = j >> 6;
    unsigned long long bits = sMask[wi] & (~0ull << (j & 63));
    while (bits == 0ull) {
      if (++wi << 6 >= n_off) return n_off;
      bits = sMask[wi];
    }
    return min((wi << 6) + (int)__builtin_ctzll(bits), n_off);
  };

  RowState st;
  st.mt = kNegInf;
  st.mref = kNegInf;
  st.l = 0.f;
  f32x16 o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[md][v] = 0.f;

  // Gate statistic of each row of this wave for tile j, in raw score units (the scale is applied
  // at the decision): the row max for ABSOLUTE and DENSE and for the diagonal region in every
  // mode; for RELATIVE off-diagonal tiles, row max - running max (-inf for rows past N). Lanes
  // l and l + 32 hold the same row and store the same value.
  auto publish = [&](int j, float rmax, float* slot) {
    float x;
    if (GATE == kRelative && j < n_off)
      x = rvalid ? rmax - st.mt : kNegInf;
    else
      x = rmax;
    slot[w * kRows + (lane & 31)] = x;
  };

  // ---- prologue: the first two tiles of the sequence staged, scores of the first published ----
  // (both copies in flight together, so the first barrier costs one memory round trip; the
  // wait covers the Q rows as well)
  int t = next_tile(-1);
  int t1 = next_tile(t);
  load_k(t, lK0);
  if (t1 < n_end) load_k(t1, lK1);
  wait_vmem();
  __syncthreads();
  f32x16 sb[2][2];     // scores of the last tiles of each parity
  float rc;            // row max of the newest scores
  qk32<D>(sK0, qf, sb[0], lane);
  rc = rowmax32(sb[0], tile_masked(t), t * BK, arow, rvalid, lane);
  if (want_stat) publish(t, rc, sGate[0]);
  wait_vmem();
  __syncthreads();

  bool keep_prev = false;
  bf16x8 pb[2][4];     // P of the last tiles of each parity; PV of the previous tile reads pb[P ^ 1]
  const int kfo = (lane & 31) * STR + 8 * (lane >> 5);
  constexpr int NSTEP = 4 * MD;               // PV MFMA steps
  // PV steps issued before the decision on tile t: all of them in the voting kernels; dense
  // and the mask walk decide nothing and start tile t's exponentials after two
  constexpr int DEC = (GATE == kRelative || GATE == kAbsVote) ? NSTEP : 2;
  constexpr int GV = WPH * kRows / 64;        // statistics per lane per head
  constexpr int MKR = copy_iters<STR, NW>(), MVR = copy_iters<STRV, NW>();

  // One iteration over sequence position u (P = u & 1 picks the LDS, P and score buffers) with
  // tile t and the next two tiles t1, t2 of the sequence:
  //   PV phase: the PV product of the previous tile (if kept). Dense and the mask walk run the
  //     V_t copy and half of tile t's exponentials next to its MFMAs. The voting kernels (the
  //     relative gate, the absolute gate decided in the loop) read the per-row statistics of
  //     tile t meanwhile and vote after the phase (keep iff some row's statistic reaches the
  //     threshold);
  //   QK phase: scores of tile t1 with the K_{t2} copy, the rest of tile t's exponentials (in
  //     the voting kernels all of them, none if t is skipped, and the V_t copy if some head of
  //     the workgroup keeps t) and the first half of t1's row max next to the MFMAs; then t1's
  //     statistics are published and the one barrier makes them and both copies visible.
  // The last iteration computes scores of a tile past the end from stale LDS and discards them,
  // which keeps the loop body free of branches around the MFMAs.
  auto body = [&](auto par) {
    constexpr int P = decltype(par)::value;
    const int t2 = next_tile(t1);
    const bool diag = t >= n_off;
    float gv[HPW][GV];
    if (want_stat) {
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const float* gp = sGate[P] + hh * WPH * kRows + GV * lane;
        if constexpr (GV == 2) {
          const float2 x = *reinterpret_cast<const float2*>(gp);
          gv[hh][0] = x.x;
          gv[hh][GV - 1] = x.y;
        } else {
          gv[hh][0] = gp[0];
        }
      }
    }
    const bool kload = t2 < n_end;
    const __bf16* const kg = Kb + tile_offset<PAGED>(a, b, min(t2, n_end - 1), kst, a.ks[0]);
    const __bf16* const vg = Vb + tile_offset<PAGED>(a, b, t, vst, a.vs[0]);
    // Whole tiles are copied by lean rounds interleaved with the MFMAs; a ragged tile (the
    // last key tile of a sequence whose length is not a multiple of 64) in one piece after the
    // phase that would have carried it, with its rows past the end redirected (copy_tile).
    const bool kfast = kload && key_valid(t2) == BK;
    const bool vfast = key_valid(t) == BK;
    auto copy_k = [&](int r) { copy_round_full<D, STR, NW>(r, koff, kg, P ? lK1 : lK0, w); };
    // V_t copy rounds: tested per round in dense and the walk; the voting kernels' forms that
    // issue them run only when tile t is whole
    auto copy_v_tested = [&](int r) {
      if (vfast) copy_round_full<D, STRV, NW>(r, voff, vg, P ? lV1 : lV0, w);
    };
    auto copy_v = [&](int r) { copy_round_full<D, STRV, NW>(r, voff, vg, P ? lV1 : lV0, w); };
    auto copy_v_ragged = [&]() {
      if (!vfast) copy_tile<D, STRV, NW>(voff, vg, vrow, key_valid(t), P ? lV1 : lV0, w, lane);
    };
    const __bf16* const sv = P ? sV0 : sV1;     // V of the previous tile
    bf16x8 vb[3];
    float sum = 0.f;
    // this tile's P buffer was last read by the previous iteration's PV: its old contents are
    // dead (a skipped tile leaves it unwritten, and then the next PV does not read it)
#pragma unroll
    for (int k = 0; k < 4; ++k) asm("" : "=v"(pb[P][k]));
    // The reference update of tile t, made before the vote into a copy: the exponentials
    // need its offset and would otherwise wait for the statistics' LDS round trip and the
    // vote. A skipped tile leaves the state as it was (its exponentials are computed and not
    // used); a kept one takes the copy, so the arithmetic is the same either way.
    RowState sp = st;
    float alpha = 1.f;
    bool moved = update_reference(sp, rc, c, alpha);
    const float off = -sp.mref * c;
    constexpr bool kVote = GATE == kRelative || GATE == kAbsVote;
    // The voting kernels run the whole PV phase of the previous tile first (the statistics'
    // LDS read lands meanwhile), then vote; dense and the mask walk keep every tile they visit
    // and start tile t's exponentials and V copy after the first PV steps.
    if (keep_prev) {
      pv_prefetch<D>(sv, vb, lane);
      pv_steps<D, 0, DEC, DEC, MVR>(true, false, false, sv, pb[P ^ 1], o, vb, sb[P], 0.f, c,
                                    pb[P], sum, lane, copy_v);
    }

    bool mykeep = true, anyv = true;
    if (want_stat) {
      float hv[HPW];
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        float x = gv[hh][0];
#pragma unroll
        for (int k = 1; k < GV; ++k) x = fmaxf(x, gv[hh][k]);
        hv[hh] = x * a.scale;
      }
      if (loop_gate && !diag) {
        anyv = false;
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          const bool k = __any(hv[hh] >= thr[hh]);
          anyv |= k;
          if (hh == hw) mykeep = k;
        }
      }
      if (a.dbg) {
        float x = hv[0];
#pragma unroll
        for (int hh = 1; hh < HPW; ++hh) x = hh == hw ? hv[hh] : x;
        x = wave_max(x);
        if (head_leader) a.dbg[(((long long)b * a.Hq + h) * a.nqb + i) * a.nkb + t] = x;
      }
    }
    if (loop_gate && head_leader && !diag) kept += mykeep ? 1 : 0;

    if (mykeep)
      st = sp;
    else
      moved = false;
    // Rest of the PV phase (dense and the mask walk) with the first kPairsPV exponential pairs
    // of tile t and the V_t copy, in straight-line forms (and a flagged one for the first tile).
    if constexpr (!kVote) {
      if (keep_prev)
        pv_steps<D, DEC, NSTEP, DEC, MVR, kAlways, kAlways, kAlways>(
            true, true, true, sv, pb[P ^ 1], o, vb, sb[P], off, c, pb[P], sum, lane,
            copy_v_tested);
      else
        pv_steps<D, DEC, NSTEP, DEC, MVR, kNever, kAlways, kAlways>(
            false, true, true, sv, pb[P ^ 1], o, vb, sb[P], off, c, pb[P], sum, lane,
            copy_v_tested);
      copy_v_ragged();
    }
    // the previous P is dead from here on (the next write of its buffer precedes the next read)
#pragma unroll
    for (int k = 0; k < 4; ++k) asm("" : "=v"(pb[P ^ 1][k]));
    // a reference move at tile t rescales O after the previous PV and before PV of tile t
    if (moved) {
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[md][v] *= alpha;
      st.l *= alpha;
    }

    // Scores of tile t1 with the K_{t2} copy, the remaining exponentials of tile t and the
    // first half of t1's row max next to the MFMAs. In the voting kernels this phase also
    // carries all of tile t's exponentials, left out when t is skipped (a skipped tile
    // computes no exponentials, "Skipping attention blocks was the easy part", Vote, then
    // skip), and the V_t copy, made when some head of the workgroup keeps t. One form per
    // combination, chosen once per phase.
    const __bf16* const kb = (P ? sK0 : sK1) + kfo;   // K of t1
    float mx = kNegInf;
    constexpr int NPV = kVote ? 0 : kPairsPV;
    // the V_t copy in the voting kernels: with one head per workgroup some head keeps t
    // exactly when this one does, so each form copies always or never; with more heads a flag
    constexpr int VQK = kVote ? (HPW == 1 ? kAlways : kFlag) : kNever;   // t kept here
    constexpr int VQS = kVote ? (HPW == 1 ? kNever : kFlag) : kNever;    // t skipped here
    // (the straight-line forms need whole tiles: K_{t2} copied in rounds, and in the voting
    // kernels V_t as well; otherwise a form with flags, the ragged tile copied after it)
    constexpr int VQG = kVote ? kFlag : kNever;
    constexpr int KLG = kVote ? kFlag : kNever;   // (dense and the walk: only when K is ragged)
    const bool vq = anyv && vfast;
    if (!kVote || mykeep) {
      if (kfast && (!kVote || vfast))
        qk_phase<D, MKR, kAlways, kAlways, NPV, MVR, VQK>(true, true, kb, qf, sb[P ^ 1], sb[P],
                                                          off, c, pb[P], sum, mx, copy_k, vq,
                                                          copy_v);
      else
        qk_phase<D, MKR, kAlways, KLG, NPV, MVR, VQG>(true, kfast, kb, qf, sb[P ^ 1], sb[P],
                                                        off, c, pb[P], sum, mx, copy_k, vq,
                                                        copy_v);
    } else {
      if (kfast)
        qk_phase<D, MKR, kNever, kAlways, NPV, MVR, VQS>(false, true, kb, qf, sb[P ^ 1], sb[P],
                                                         off, c, pb[P], sum, mx, copy_k, vq,
                                                         copy_v);
      else
        qk_phase<D, MKR, kNever, kFlag, NPV, MVR, VQS>(false, false, kb, qf, sb[P ^ 1], sb[P],
                                                       off, c, pb[P], sum, mx, copy_k, vq,
                                                       copy_v);
    }
    if (kload && !kfast) load_k(t2, P ? lK1 : lK0);
    if constexpr (kVote) {
      if (anyv) copy_v_ragged();
    }
    if (mykeep) st.l += sum;
    if (tile_masked(t1)) {
      mask_tile(sb[P ^ 1], t1 * BK, arow, rvalid, lane);
      mx = kNegInf;
#pragma unroll
      for (int v = 0; v < 16; v += 2) mx = max3(mx, sb[P ^ 1][0][v], sb[P ^ 1][0][v + 1]);
    }
    mx = block_max(mx, sb[P ^ 1][1]);
    rc = half_max(mx);
    if (want_stat) publish(t1, rc, sGate[P ^ 1]);
    wait_vmem();
    __syncthreads();
    keep_prev = mykeep;
    t = t1;
    t1 = t2;
  };

  // sequence length: the kept off-diagonal tiles (all of them without the pass-1 mask) and the
  // diagonal region
  const int n_seq = (two_pass ? kept_all : n_off) + (n_end - n_off);
  int u = 0;
  for (; u + 1 < n_seq; u += 2) {
    body(IC<0>{});
    body(IC<1>{});
  }
  if (u < n_seq) body(IC<0>{});
  const int last = (n_seq - 1) & 1;   // parity of the last sequence position

  if (keep_prev) {   // always: the last tile is diagonal
    float dsum = 0.f;
    bf16x8 dummy[4], vb[3];
    const __bf16* const sv = last ? sV1 : sV0;
    pv_prefetch<D>(sv, vb, lane);
    if (last)
      pv_steps<D, 0, NSTEP, NSTEP, 1>(true, false, false, sv, pb[1], o, vb, sb[0], 0.f, c,
                                      dummy, dsum, lane, [](int) {});
    else
      pv_steps<D, 0, NSTEP, NSTEP, 1>(true, false, false, sv, pb[0], o, vb, sb[0], 0.f, c,
                                      dummy, dsum, lane, [](int) {});
  }

  if constexpr (MEAN) {
    // ---- mean correction ("FlashPrefill V2", mean correction) ----
    // A pruned gate block J enters the softmax as one more key: its mean key, with the logit
    // shifted by ln(block keys), and its mean value, i.e. |B| e^{s(q, kbar)} joins l and
    // |B| e^{s(q, kbar)} vbar joins O. 64 such pseudo-keys (blocks m0 .. m0 + 63) make a tile:
    // scored against Q by MFMAs over the mean key's bf16 high and low parts in turn, masked
    // where the block was kept or does not exist, then the online-softmax update and the PV
    // product of a key tile. Blocks are whole here: off-diagonal blocks never reach the end.
    // (The walk has drained: its last barrier waited for every copy.)
    if (two_pass && kept_all < n_off) {
      const int n_gb = min(n_off / a.kpb, a.mean_blocks);
      const long long mbase = ((long long)b * a.Hkv + g) * a.mean_blocks * D;
      const __bf16* const khi = static_cast<const __bf16*>(a.kbar_hi) + mbase;
      const __bf16* const klo = static_cast<const __bf16*>(a.kbar_lo) + mbase;
      const __bf16* const vme = static_cast<const __bf16*>(a.vbar) + mbase;
      unsigned mko[MK], mvo[MV];
      copy_offsets<D, STR, NW>(mko, D, w, lane);
      copy_offsets<D, STRV, NW>(mvo, D, w, lane);
      const int hs = lane >> 5;
      // mean tile m0 (pseudo-keys m0 .. m0 + 63): k-bar parts in sK0 / sK1, v-bar in sV0 or
      // sV1 by parity. The next tile's v-bar is copied into the other V buffer during this
      // tile's scores, and its k-bar parts once every wave has read this tile's (a second
      // barrier), during the exponentials and the PV product.
      auto stage_k = [&](int m) {
        const int valid = min(64, n_gb - m);
        copy_tile<D, STR, NW>(mko, khi + (long long)m * D, 2u * D, valid, lK0, w, lane);
        copy_tile<D, STR, NW>(mko, klo + (long long)m * D, 2u * D, valid, lK1, w, lane);
      };
      auto stage_v = [&](int m, unsigned dst) {
        copy_tile<D, STRV, NW>(mvo, vme + (long long)m * D, 2u * D, min(64, n_gb - m), dst, w,
                               lane);
      };
      __syncthreads();   // every wave is done with the walk's tile buffers
      stage_k(0);
      stage_v(0, lV0);
      bool par = false;
      for (int m0 = 0; m0 < n_gb; m0 += 64, par = !par) {
        __bf16* const sv = par ? sV1 : sV0;
        const bool more = m0 + 64 < n_gb;
        wait_vmem();
        __syncthreads();   // tile m0 visible; every wave is done with the other V buffer
        if (more) stage_v(m0 + 64, par ? lV0 : lV1);
        // S^T of the pseudo-keys: the high and low parts into one accumulator
        f32x16 sm[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int v = 0; v < 16; ++v) sm[mb][v] = 0.f;
        const int kro = (lane & 31) * STR + 8 * (lane >> 5);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            const int ko = kro + mb * 32 * STR + 16 * ks;
            sm[mb] = mfma32(*reinterpret_cast<const bf16x8*>(sK0 + ko), qf[ks], sm[mb]);
            sm[mb] = mfma32(*reinterpret_cast<const bf16x8*>(sK1 + ko), qf[ks], sm[mb]);
          }
        __syncthreads();   // every wave has read this tile's k-bar parts
        if (more) stage_k(m0 + 64);
        float mx = kNegInf;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int J = m0 + mb * 32 + 8 * (v >> 2) + 4 * hs + (v & 3);
            const int t0 = J * a.kpb;   // a kept block sets the bits of all its tiles
            const bool pruned =
                rvalid && J < n_gb && !((sMask[t0 >> 6] >> (t0 & 63)) & 1ull);
            const float x = pruned ? sm[mb][v] + a.mean_bias : kNegInf;
            sm[mb][v] = x;
            mx = fmaxf(mx, x);
          }
        float alpha = 1.f;
        if (update_reference(st, half_max(mx), c, alpha)) {
#pragma unroll
          for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[md][v] *= alpha;
          st.l *= alpha;
        }
        bf16x8 pm[4], vb[3], dummy[4];
        float sum = 0.f, dsum = 0.f;
#pragma unroll
        for (int pi = 0; pi < kPairs; ++pi) exp_pair(pi, sm, -st.mref * c, c, pm, sum);
        st.l += sum;
        pv_prefetch<D>(sv, vb, lane);
        pv_steps<D, 0, NSTEP, NSTEP, 1>(true, false, false, sv, pm, o, vb, sm, 0.f, c, dummy,
                                        dsum, lane, [](int) {});
      }
    }
  }

  // ---- epilogue: O / l (renormalised over kept + diagonal), kept counts ----
  const int hh = lane >> 5;
  const float inv = 1.f / half_sum(st.l);
  if (row < N) {
    const long long base = sq.o + (long long)row * a.os[1] + h * a.os[2];
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = md * 32 + 8 * q4 + 4 * hh;
        const float x0 = o[md][4 * q4 + 0] * inv, x1 = o[md][4 * q4 + 1] * inv;
        const float x2 = o[md][4 * q4 + 2] * inv, x3 = o[md][4 * q4 + 3] * inv;
        if (a.out_fp32) {
          *reinterpret_cast<float4*>(static_cast<float*>(a.o) + base + d0) =
              make_float4(x0, x1, x2, x3);
        } else {
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
  if (head_leader) {
    if (a.kept_counts) a.kept_counts[((long long)b * a.Hq + h) * a.nqb + i] = kept;
    if (a.kept_total) atomicAdd(a.kept_total, (unsigned long long)kept);
  }
  if (kLoop && tickets) {
    __syncthreads();   // every wave is done with this unit's LDS (and has read sUnit)
    goto next_unit;
  }
}


// ---------------------------------------------------------------------------------------------
// Gate sweep (absolute gate; launched before the prefill kernel): for every (b, h, i) the
// maxima of all off-diagonal tiles, two tiles per barrier, compared with T_eff(h, i); kept
// tiles set their bit in the keep mask. Every workgroup does the same work per tile, so the
// workgroups that share a KV head stream its K tiles in step and mostly from L2; the
// workgroup's heads share each staged K tile. With no softmax state to hold, a wave takes 64
// query rows: each K fragment read from LDS feeds two MFMAs, which halves the LDS reads per
// product (32-row waves read K from LDS as fast as the MFMAs consume it).
// ---------------------------------------------------------------------------------------------

// S^T for one 64-key tile and 64 query rows (two 32-row halves rb): s[rb][mb] as in qk32 for
// rows row0 + 32 rb. Same k-step order as qk32, so every score is bitwise the same.
template <int D>
__device__ __forceinline__ void qk64(const __bf16* sk, const bf16x8 (&qf)[2][D / 16],
                                     f32x16 (&s)[2][2], int lane) {
  constexpr int KS = Tile<D>::KS, STR = Tile<D>::STR;
  const __bf16* base = sk + (lane & 31) * STR + 8 * (lane >> 5);
  bf16x8 ka[2][2];
  auto load = [&](int ks, int buf) {
    ka[buf][0] = *reinterpret_cast<const bf16x8*>(base + 16 * ks);
    ka[buf][1] = *reinterpret_cast<const bf16x8*>(base + 32 * STR + 16 * ks);
  };
  load(0, 0);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < KS) load(ks + 1, buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        if (ks == 0) {
          f32x16 z;
#pragma unroll
          for (int v = 0; v < 16; ++v) z[v] = 0.f;
          s[rb][mb] = mfma32(ka[buf][mb], qf[rb][ks], z);
        } else {
          s[rb][mb] = mfma32(ka[buf][mb], qf[rb][ks], s[rb][mb]);
        }
      }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// This lane's max over a fully visible tile's scores for the wave's 64 rows; rows at or past
// N (the last query block only) do not count.
__device__ __forceinline__ float tile_max64(f32x16 (&s)[2][2], bool ragged, int row0, int N,
                                            int lane) {
  if (ragged) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      if (row0 + 32 * rb + (lane & 31) >= N)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int v = 0; v < 16; ++v) s[rb][mb][v] = kNegInf;
  }
  float mx = block_max(kNegInf, s[0][0]);
  mx = block_max(mx, s[0][1]);
  mx = block_max(mx, s[1][0]);
  return block_max(mx, s[1][1]);
}

// Copy whole key tile j of the sweep (all rounds of this wave) into the LDS buffer at byte
// address dst.
template <int D, int NW, bool PAGED>
__device__ __forceinline__ void sweep_load_k(const PrefillArgs& a, int b, int j, const __bf16* Kb,
                                             long long kst,
                                             const unsigned (&koff)[copy_iters<Tile<D>::STR, NW>()],
                                             unsigned dst, int w) {
  constexpr int STR = Tile<D>::STR, MK = copy_iters<STR, NW>();
  const __bf16* const g = Kb + tile_offset<PAGED>(a, b, j, kst, a.ks[0]);
  // (the wave index opaque here: otherwise the last round's test is computed once per kernel
  // and held, under this kernel's register pressure, in a spilled vector register whose reload
  // waits for every copy in flight)
  int wc = w;
  asm volatile("" : "+s"(wc));
#pragma unroll
  for (int m = 0; m < MK; ++m) copy_round_full<D, STR, NW>(m, koff, g, dst, wc);
}

template <int D, int BQ, int HPW, bool PAGED>
__global__ __launch_bounds__(HPW * (BQ / 64) * 64) __attribute__((amdgpu_waves_per_eu(3, 3)))
void gate_sweep_kernel(PrefillArgs a) {
  constexpr int WPH = BQ / 64;             // waves per head
  constexpr int NW = HPW * WPH;
  constexpr int STR = Tile<D>::STR, KS = Tile<D>::KS;
  constexpr int MK = copy_iters<STR, NW>(), CPS = STR / 8;

  // three K tiles: tile j is read from buffer j % 3 while tiles j + 1 and j + 2 are in flight
  __shared__ __attribute__((aligned(16))) __bf16 sKa[64 * STR];
  __shared__ __attribute__((aligned(16))) __bf16 sKb[64 * STR];
  __shared__ __attribute__((aligned(16))) __bf16 sKc[64 * STR];
  __shared__ float sStage[2][NW];

  __shared__ int sUnit;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = w / WPH, rw = w % WPH;
  // one unit (b, KV head, head pair, query block) at place L of the unit order
  auto run_unit = [&](const int L) __attribute__((always_inline)) {
  const Unit un = decode_unit(L, a.units, a.nqb, a.B, a.Hkv, a.xcd_map, a.xcd_rot);
  const int b = un.b, g = un.g, i = un.i;
  const int h0 = g * a.G + un.hg * HPW;
  const int h = h0 + hw;
  const Seq sq = seq_of(a, b);   // query rows at absolute positions pre .. (see prefill_kernel)
  if (i * BQ >= sq.N) return;     // uniform: past this sequence's query blocks (variable length)
  const int N = sq.N, pre = sq.pre;
  const int row0 = i * BQ + rw * 64;
  const int n_off = (pre + i * BQ) / BK;
  const bool ragged_rows = (i + 1) * BQ > N;
  const bool leader = rw == 0 && lane == 0;   // one lane per head: its decisions and mask words
  unsigned long long* const mask = a.keep_mask + (((long long)b * a.Hq + h) * a.nqb + i) *
                                                     a.mask_words;
  // with full_masks every word of every head is written (zero past the off-diagonal tiles)
  const int nw64 = (n_off + 63) >> 6;
  auto zero_tail = [&]() {
    if (a.full_masks && leader)
      for (int x = nw64; x < a.mask_words; ++x) mask[x] = 0ull;
  };
  if (n_off == 0) {         // uniform: nothing off-diagonal to decide
    zero_tail();
    return;
  }

  const __bf16* Qb = static_cast<const __bf16*>(a.q) + sq.q + h * a.qs[2];
  const __bf16* Kb = static_cast<const __bf16*>(a.k) + sq.k + g * a.ks[2];
  const long long kst = a.ks[1];
  unsigned koff[MK];
  copy_offsets<D, STR, NW>(koff, kst, w, lane);
  // off-diagonal key tiles are whole: every round is a plain copy to a precomputed LDS address
  const unsigned lKa = lds_addr(sKa), lKb = lds_addr(sKb), lKc = lds_addr(sKc);
  auto kbuf = [&](int x) { return x == 0 ? sKa : x == 1 ? sKb : sKc; };
  const int tcol = min(pre / BQ + i, a.t_len - 1);   // the absolute query block's threshold
  const float thr = a.thr[h * a.t_len + tcol];
  // heads whose threshold is -inf keep everything without a mask (the softmax kernel does not
  // read one then), so a workgroup of only such heads has nothing to decide unless the maxima
  // are dumped
  bool all_keep = a.dbg == nullptr && !a.full_masks;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
    all_keep = all_keep && a.thr[(h0 + hh) * a.t_len + tcol] == kNegInf;
  if (all_keep) return;

  // The copy instructions one tile takes from this wave (the last round only on some waves):
  // waiting until that many remain outstanding leaves the newest tile in flight.
  const bool last_round = w + NW * (MK - 1) < CPS;
  auto wait_all_but_newest_tile = [&]() {
    if (last_round)
      wait_vmem_n<MK>();
    else
      wait_vmem_n<MK - 1>();
  };
  // leader of head hw: decision for tile j from the head's waves' maxima in slot j & 1; each
  // completed mask word goes out at once
  // (with 128-key gate blocks, a block is decided on its second tile from both tiles' maxima
  // and keeps both bits; n_off is a whole number of blocks then, since BQ = 128)
  unsigned long long word = 0ull;
  float xblk = kNegInf;
  auto combine = [&](int j) {
    if (leader) {
      float x = sStage[j & 1][hw * WPH];
#pragma unroll
      for (int r = 1; r < WPH; ++r) x = fmaxf(x, sStage[j & 1][hw * WPH + r]);
      xblk = (j % a.kpb == 0) ? x : fmaxf(xblk, x);
      if (j % a.kpb == a.kpb - 1) {
        const int jb = j / a.kpb;
        const float sm = xblk * a.scale;
        if (a.dbg) a.dbg[(((long long)b * a.Hq + h) * a.nqb + i) * a.nkb + jb] = sm;
        if (sm >= thr) word |= (a.kpb == 2 ? 3ull : 1ull) << ((j + 1 - a.kpb) & 63);
      }
      if ((j & 63) == 63 || j == n_off - 1) {
        mask[j >> 6] = word;
        word = 0ull;
      }
    }
  };

  sweep_load_k<D, NW, PAGED>(a, b, 0, Kb, kst, koff, lKa, w);
  if (n_off > 1) sweep_load_k<D, NW, PAGED>(a, b, 1, Kb, kst, koff, lKb, w);
  bf16x8 qf[2][KS];
  load_q32<D>(Qb, a.qs[1], row0, N, qf[0], lane);
  load_q32<D>(Qb, a.qs[1], row0 + 32, N, qf[1], lane);
  wait_vmem();
  __syncthreads();
  for (int j = 0; j < n_off; ++j) {
    if (j + 2 < n_off) {   // into the buffer tile j - 1 used
      const int x = (j + 2) % 3;
      sweep_load_k<D, NW, PAGED>(a, b, j + 2, Kb, kst, koff, x == 0 ? lKa : x == 1 ? lKb : lKc, w);
    }
    f32x16 s[2][2];
    qk64<D>(kbuf(j % 3), qf, s, lane);
    const float m = wave_max(tile_max64(s, ragged_rows, row0, N, lane));
    if (lane == 0) sStage[j & 1][w] = m;
    if (j > 0) combine(j - 1);
    // tile j + 1 must have landed before the barrier; tile j + 2 may stay in flight
    if (j + 2 < n_off)
      wait_all_but_newest_tile();
    else
      wait_vmem();
    __syncthreads();
  }
  combine(n_off - 1);
  zero_tail();
  };

  // Workgroup L runs unit L; with ticket counters (zero at the launch) the launch holds the
  // workgroups resident at once and each takes units in turn until none is left, so that the
  // XCDs, whose speeds differ by a few per cent under this load, share the work as they go.
  // With the XCD assignment (xcd_map = 1: unit place L belongs to XCD L mod 8, one KV head per
  // XCD when B * Hkv = 8), each XCD has its own queue, the places L = 8 t + x in order of t,
  // so that its workgroups stream one K sequence through its L2; a workgroup takes from its
  // own XCD's queue (the XCC_ID register) and, once that is empty, from the others'. Otherwise
  // one counter hands out every place in turn.
  if (a.ticket) {
    const int U = a.units * a.nqb;
    int q = a.xcd_map == 1 ? (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 7) : 0;
    for (;;) {
      if (tid == 0) {
        int L = -1;
        if (a.xcd_map == 1) {
          for (int k = 0; k < 8 && L < 0; ++k) {   // the queue in hand first, then the others
            const int y = (q + k) & 7;
            const int t = (int)atomicAdd(a.ticket + y, 1u);
            if (t < (U - y + 7) / 8) {
              L = 8 * t + y;
              q = y;
            }
          }
        } else {
          const int t = (int)atomicAdd(a.ticket, 1u);
          L = t < U ? t : -1;
        }
        sUnit = L;
      }
      __syncthreads();
      const int L = __builtin_amdgcn_readfirstlane(sUnit);
      if (L < 0) break;   // uniform: every unit taken
      run_unit(L);
      __syncthreads();   // every wave is done with this unit's LDS (and has read sUnit)
    }
  } else {
    run_unit(blockIdx.x);
  }
}

// ---------------------------------------------------------------------------------------------
// FP8 (E4M3) gate scores. Q is quantised per (token, head) row and K per (64-key tile, KV head):
// scale = amax / 448, codes = x * (448 / amax) rounded to nearest even on the E4M3 grid (the
// hardware conversion; the product is clamped to +-448 first, so nothing saturates), in fp32;
// an all-zero row or tile gets codes 0 and scale 0. The copies are dense:
// q8 [B][q8_rows][Hq][D] with scales [B][Hq][q8_rows], k8 [B][k8_rows][Hkv][D] with scales
// [B][Hkv][k8_tiles], whatever the layout of Q and K (strided, packed or paged).
// ---------------------------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) int i32x8;

// Four fp32 values as four E4M3 codes in one 32-bit word (value k in byte k).
__device__ __forceinline__ unsigned pack_e4m3(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return (unsigned)w;
}

__device__ __forceinline__ float e4m3_inv(float amax) {
  return amax > 0.f ? __fdiv_rn(448.f, amax) : 0.f;
}
__device__ __forceinline__ float e4m3_scale(float amax) {
  return amax > 0.f ? __fdiv_rn(amax, 448.f) : 0.f;
}

// Eight bf16 values times inv, clamped to +-448, as eight codes.
__device__ __forceinline__ uint2 quant8(const bf16x8& x, float inv) {
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf((float)x[e] * inv, -448.f), 448.f);
  return make_uint2(pack_e4m3(y[0], y[1], y[2], y[3]), pack_e4m3(y[4], y[5], y[6], y[7]));
}

__device__ __forceinline__ float amax8(const bf16x8& x) {
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)x[e]));
  return m;
}

// One (token, head) row of Q per D/8 lanes; 256 threads hold 4 * 64 / (D/8) rows.
template <int D>
__global__ __launch_bounds__(256) void quant_q_kernel(PrefillArgs a) {
  constexpr int LPR = D / 8, RPW = 64 / LPR, RPB = 4 * RPW;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int per = (a.q8_rows * a.Hq + RPB - 1) / RPB;    // workgroups per sequence
  const int b = blockIdx.x / per;
  const int u = (blockIdx.x % per) * RPB + w * RPW + lane / LPR;
  const Seq sq = seq_of(a, b);
  const int r = u / a.Hq, h = u % a.Hq;
  if (r >= sq.N) return;                       // whole row groups leave together
  const int col = (lane % LPR) * 8;
  const bf16x8 x = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.q) + sq.q +
                                                     (long long)r * a.qs[1] + h * a.qs[2] + col);
  float m = amax8(x);
#pragma unroll
  for (int s = 1; s < LPR; s <<= 1) m = fmaxf(m, __shfl_xor(m, s));
  const long long row = (long long)b * a.q8_rows + r;
  *reinterpret_cast<uint2*>(static_cast<unsigned char*>(a.q8) + (row * a.Hq + h) * D + col) =
      quant8(x, e4m3_inv(m));
  if (lane % LPR == 0)
    a.q8_scale[((long long)b * a.Hq + h) * a.q8_rows + r] = e4m3_scale(m);
}

// One (64-key tile, KV head) of K per workgroup of 256 threads.
template <int D, bool PAGED>
__global__ __launch_bounds__(256) void quant_k_kernel(PrefillArgs a) {
  constexpr int LPR = D / 8, CH = 64 * LPR / 256;    // 8-element chunks per thread
  __shared__ float sAmax[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t = blockIdx.x % a.k8_tiles;
  const int bg = blockIdx.x / a.k8_tiles;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const Seq sq = seq_of(a, b);
  if (t * kBlockK >= sq.Nk) return;                  // uniform: past this sequence's keys
  const int valid = min(kBlockK, sq.Nk - t * kBlockK);
  const long long kst = a.ks[1];
  const __bf16* const Kt = static_cast<const __bf16*>(a.k) + sq.k + g * a.ks[2] +
                           tile_offset<PAGED>(a, b, t, kst, a.ks[0]);
  bf16x8 x[CH];
  float m = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int q = tid + 256 * c, r = q / LPR;
    if (r < valid) {
      x[c] = *reinterpret_cast<const bf16x8*>(Kt + (long long)r * kst + (q % LPR) * 8);
      m = fmaxf(m, amax8(x[c]));
    }
  }
  m = wave_max(m);
  if (lane == 0) sAmax[w] = m;
  __syncthreads();
  m = fmaxf(fmaxf(sAmax[0], sAmax[1]), fmaxf(sAmax[2], sAmax[3]));
  const float inv = e4m3_inv(m);
  unsigned char* const out = static_cast<unsigned char*>(a.k8) +
                             (((long long)b * a.k8_rows + t * kBlockK) * a.Hkv + g) * D;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int q = tid + 256 * c, r = q / LPR;
    if (r < valid)
      *reinterpret_cast<uint2*>(out + (long long)r * a.Hkv * D + (q % LPR) * 8) = quant8(x[c], inv);
  }
  if (tid == 0) a.k8_scale[((long long)b * a.Hkv + g) * a.k8_tiles + t] = e4m3_scale(m);
}

// The gate sweep on FP8 scores: the structure of gate_sweep_kernel (three K tiles in LDS, one
// per barrier, 64-row waves, the heads of a KV group sharing each tile), with E4M3 Q and K and
// v_mfma_scale_f32_32x32x64_f8f6f4 at unit block scales: a 64-row wave takes D/64 k-steps of
// four MFMAs per tile (32 bf16 ones at d = 128). A lane holds 32 consecutive bytes of its row
// per operand (lanes 32..63 the second 32 of each 64); both operands use the same order, which
// is all a dot product needs. The row maximum of the raw dot products is scaled by the row's
// Q scale, the tile maximum by the tile's K scale and the softmax scale.
// LDS K rows: D bytes + 16 of padding, so that 16 rows start 36 banks apart and a 16-byte read
// of 16 rows covers the 64 banks once. At d = 128 a wave needs 126 VGPRs (Q fragments 32,
// scores 64), so four waves share a SIMD (one more than the bf16 sweep): 7 % faster.
template <int D, int BQ, int HPW>
__global__ __launch_bounds__(HPW * (BQ / 64) * 64) __attribute__((amdgpu_waves_per_eu(4, 4)))
void gate_sweep_fp8_kernel(PrefillArgs a) {
  constexpr int WPH = BQ / 64;
  constexpr int NW = HPW * WPH;
  constexpr int D2 = D / 2, STR8 = D2 + 8;     // a row in 2-byte units: D bytes + 16 of padding
  constexpr int KS8 = D / 64;                  // k-steps of 64 bytes
  constexpr int MK = copy_iters<STR8, NW>(), CPS = STR8 / 8;

  __shared__ __attribute__((aligned(16))) __bf16 sKa[64 * STR8];
  __shared__ __attribute__((aligned(16))) __bf16 sKb[64 * STR8];
  __shared__ __attribute__((aligned(16))) __bf16 sKc[64 * STR8];
  __shared__ float sStage[2][NW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = w / WPH, rw = w % WPH;
  const Unit un = decode_unit(blockIdx.x, a.units, a.nqb, a.B, a.Hkv, a.xcd_map, a.xcd_rot);
  const int b = un.b, g = un.g, i = un.i;
  const int h0 = g * a.G + un.hg * HPW;
  const int h = h0 + hw;
  const Seq sq = seq_of(a, b);
  if (i * BQ >= sq.N) return;
  const int N = sq.N, pre = sq.pre;
  const int row0 = i * BQ + rw * 64;
  const int n_off = (pre + i * BQ) / BK;
  const bool leader = rw == 0 && lane == 0;
  unsigned long long* const mask = a.keep_mask + (((long long)b * a.Hq + h) * a.nqb + i) *
                                                     a.mask_words;
  const int nw64 = (n_off + 63) >> 6;
  auto zero_tail = [&]() {
    if (a.full_masks && leader)
      for (int x = nw64; x < a.mask_words; ++x) mask[x] = 0ull;
  };
  if (n_off == 0) {
    zero_tail();
    return;
  }

  // K tiles of this (b, g) in the dense FP8 copy, addressed in 2-byte units for the copies
  const long long kst2 = (long long)a.Hkv * D2;
  const __bf16* const K8 = reinterpret_cast<const __bf16*>(
      static_cast<const unsigned char*>(a.k8) + ((long long)b * a.k8_rows * a.Hkv + g) * D);
  const unsigned krow = (unsigned)(a.Hkv * D);
  unsigned koff[MK];
  copy_offsets<D2, STR8, NW>(koff, kst2, w, lane);
  const unsigned lKa = lds_addr(sKa), lKb = lds_addr(sKb), lKc = lds_addr(sKc);
  auto kbuf = [&](int x) { return x == 0 ? sKa : x == 1 ? sKb : sKc; };
  // without a table (the calibration's maxima dump) nothing is kept
  const int tcol = min(pre / BQ + i, a.t_len - 1);
  const float thr = a.thr ? a.thr[h * a.t_len + tcol] : __builtin_huge_valf();
  bool all_keep = a.thr && a.dbg == nullptr && !a.full_masks;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
    all_keep = all_keep && a.thr[(h0 + hh) * a.t_len + tcol] == kNegInf;
  if (all_keep) return;

  const bool last_round = w + NW * (MK - 1) < CPS;
  auto wait_all_but_newest_tile = [&]() {
    if (last_round)
      wait_vmem_n<MK>();
    else
      wait_vmem_n<MK - 1>();
  };
  const float* const ksc = a.k8_scale + ((long long)b * a.Hkv + g) * a.k8_tiles;
  unsigned long long word = 0ull;
  float xblk = kNegInf;
  auto combine = [&](int j) {
    if (leader) {
      float x = sStage[j & 1][hw * WPH];
#pragma unroll
      for (int r = 1; r < WPH; ++r) x = fmaxf(x, sStage[j & 1][hw * WPH + r]);
      x *= ksc[j];
      xblk = (j % a.kpb == 0) ? x : fmaxf(xblk, x);
      if (j % a.kpb == a.kpb - 1) {
        const int jb = j / a.kpb;
        const float sm = xblk * a.scale;
        if (a.dbg) a.dbg[(((long long)b * a.Hq + h) * a.nqb + i) * a.nkb + jb] = sm;
        if (sm >= thr) word |= (a.kpb == 2 ? 3ull : 1ull) << ((j + 1 - a.kpb) & 63);
      }
      if ((j & 63) == 63 || j == n_off - 1) {
        mask[j >> 6] = word;
        word = 0ull;
      }
    }
  };

  copy_tile<D2, STR8, NW>(koff, K8, krow, BK, lKa, w, lane);
  if (n_off > 1) copy_tile<D2, STR8, NW>(koff, K8 + (long long)kBlockK * kst2, krow, BK, lKb, w, lane);
  // Q rows row0 + 32 rb + lane % 32 (zero past N) and their scales
  i32x8 qf[2][KS8];
  float qs[2];
  bool rv[2];
  const unsigned char* const Q8 = static_cast<const unsigned char*>(a.q8) +
                                  ((long long)b * a.q8_rows * a.Hq + h) * D;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = row0 + 32 * rb + (lane & 31);
    rv[rb] = row < N;
    const unsigned char* p = Q8 + (long long)min(row, N - 1) * a.Hq * D + 32 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KS8; ++ks) {
      uint4 lo = *reinterpret_cast<const uint4*>(p + 64 * ks);
      uint4 hi = *reinterpret_cast<const uint4*>(p + 64 * ks + 16);
      if (!rv[rb]) lo = hi = make_uint4(0, 0, 0, 0);
      qf[rb][ks] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                         (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    qs[rb] = a.q8_scale[((long long)b * a.Hq + h) * a.q8_rows + min(row, N - 1)];
  }
  wait_vmem();
  __syncthreads();
  const int kfo = (lane & 31) * (2 * STR8) + 32 * (lane >> 5);   // byte offset in a tile
  for (int j = 0; j < n_off; ++j) {
    if (j + 2 < n_off) {   // into the buffer tile j - 1 used
      const int x = (j + 2) % 3;
      copy_tile<D2, STR8, NW>(koff, K8 + (long long)(j + 2) * kBlockK * kst2, krow, BK,
                              x == 0 ? lKa : x == 1 ? lKb : lKc, w, lane);
    }
    const unsigned char* const kt = reinterpret_cast<const unsigned char*>(kbuf(j % 3)) + kfo;
    f32x16 s[2][2];
#pragma unroll
    for (int ks = 0; ks < KS8; ++ks) {
      i32x8 kf[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const uint4 lo = *reinterpret_cast<const uint4*>(kt + mb * 32 * (2 * STR8) + 64 * ks);
        const uint4 hi = *reinterpret_cast<const uint4*>(kt + mb * 32 * (2 * STR8) + 64 * ks + 16);
        kf[mb] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          f32x16 acc;
          if (ks == 0) {
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[v] = 0.f;
          } else {
            acc = s[rb][mb];
          }
          s[rb][mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[mb], qf[rb][ks], acc,
                                                                       0, 0, 0, 127, 0, 127);
        }
    }
    float m = kNegInf;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float mr = block_max(block_max(kNegInf, s[rb][0]), s[rb][1]);
      m = fmaxf(m, rv[rb] ? mr * qs[rb] : kNegInf);
    }
    m = wave_max(m);
    if (lane == 0) sStage[j & 1][w] = m;
    if (j > 0) combine(j - 1);
    if (j + 2 < n_off)
      wait_all_but_newest_tile();
    else
      wait_vmem();
    __syncthreads();
  }
  combine(n_off - 1);
  zero_tail();
}

// ---------------------------------------------------------------------------------------------
// Calibration: per (b, h, i) the off-diagonal block maxima, then the k-th highest per budget.
// Waves of 32 rows as in the prefill kernel, QK only; the per-wave tile maxima collect in LDS.
// ---------------------------------------------------------------------------------------------
template <int D, int BQ, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void calibrate_kernel(
    CalibArgs a) {
  constexpr int NT = NW * 64;
  constexpr int WPH = BQ / kRows;
  constexpr int HPW = NW / WPH;
  constexpr int MAXJ = kCalibMaxKeyBlocks;
  constexpr int STR = Tile<D>::STR;
  constexpr int MK = copy_iters<STR, NW>();

  __shared__ __attribute__((aligned(16))) __bf16 sK[2][64 * STR];
  __shared__ float sW[HPW][MAXJ];
  __shared__ float sPart[NW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = w / WPH, rw = w % WPH;
  const Unit un = decode_unit(blockIdx.x, a.units, a.nqb, a.B, a.Hkv, a.xcd_map, a.xcd_rot);
  const int b = un.b, g = un.g, i = un.i;
  const int h0 = g * a.G + un.hg * HPW;
  const int h = h0 + hw;
  const int N = a.N;
  const int row0 = i * BQ + rw * kRows;
  const int row = row0 + (lane & 31);
  const int n_off = (i * BQ) / BK;
  const bool ragged_rows = (i + 1) * BQ > N;

  if (n_off > 0) {
    const __bf16* Qb = static_cast<const __bf16*>(a.q) + b * a.qs[0] + h * a.qs[2];
    const __bf16* Kb = static_cast<const __bf16*>(a.k) + b * a.ks[0] + g * a.ks[2];
    const long long kst = a.ks[1];
    unsigned koff[MK];
    copy_offsets<D, STR, NW>(koff, kst, w, lane);
    bf16x8 qf[D / 16];
    const unsigned krow = (unsigned)kst * 2u;
    const unsigned lK0 = lds_addr(sK[0]), lK1 = lds_addr(sK[1]);
    copy_tile<D, STR, NW>(koff, Kb, krow, BK, lK0, w, lane);
    load_q32<D>(Qb, a.qs[1], row0, N, qf, lane);
    wait_vmem();
    __syncthreads();
    for (int t = 0; t < n_off; ++t) {
      if (t + 1 < n_off)
        copy_tile<D, STR, NW>(koff, Kb + (long long)(t + 1) * BK * kst, krow, BK,
                              ((t + 1) & 1) ? lK1 : lK0, w, lane);
      f32x16 s[2];
      qk32<D>(sK[t & 1], qf, s, lane);
      const float rmax = rowmax32(s, ragged_rows, t * BK, row, row < N, lane);
      const float wst = wave_max(rmax);
      if (lane == 0) sPart[w] = wst;
      wait_vmem();
      __syncthreads();
      if (tid < HPW) {   // the candidate of gate block t / kpb: max over its tiles
        float x = sPart[tid * WPH];
        for (int r = 1; r < WPH; ++r) x = fmaxf(x, sPart[tid * WPH + r]);
        x *= a.scale;
        sW[tid][t / a.kpb] = (t % a.kpb == 0) ? x : fmaxf(sW[tid][t / a.kpb], x);
      }
      __syncthreads();
    }
  }
  // pad each head's list of gate-block candidates to a power of two with -inf, then an
  // ascending bitonic sort
  const int n_cand = n_off / a.kpb;
  int P = 1;
  while (P < n_cand) P <<= 1;
  for (int idx = tid; idx < HPW * P; idx += NT) {
    const int hh = idx / P, t = idx % P;
    if (t >= n_cand) sW[hh][t] = kNegInf;
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int idx = tid; idx < HPW * P; idx += NT) {
        const int hh = idx / P, x = idx % P, y = x ^ j;
        if (y > x) {
          float* L = sW[hh];
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
      const float r = (n_cand >= kb) ? sW[hw][P - kb] : kNegInf;
      a.kth[(((long long)kk * a.B + b) * a.Hq + h) * a.nqb + i] = r;
    }
  }
}

// k-th highest of each (b, h, i)'s off-diagonal gate-block maxima, from a dump of them
// (fp32 [B][Hq][nqb][nkb], entries j < n_off(i) / kpb valid): the list padded to a power of
// two with -inf and sorted ascending in LDS (bitonic), then one read per budget; -inf where
// fewer than k candidates exist ("Block Sparse Flash Attention", Method > Key Designs 1).
// One workgroup of 256 threads per (b, h, i).
__global__ __launch_bounds__(256) void kth_select_kernel(CalibArgs a, const float* maxima,
                                                         int block_q) {
  constexpr int MAXJ = kCalibMaxKeyBlocks;
  __shared__ float sW[MAXJ];
  const int tid = threadIdx.x;
  const int i = blockIdx.x % a.nqb, bh = blockIdx.x / a.nqb;   // bh = b * Hq + h
  const int n_cand = (i * block_q) / BK / a.kpb;
  const float* const row = maxima + ((long long)bh * a.nqb + i) * a.nkb;
  int P = 1;
  while (P < n_cand) P <<= 1;
  for (int t = tid; t < P; t += 256) sW[t] = t < n_cand ? row[t] : kNegInf;
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int x = tid; x < P; x += 256) {
        const int y = x ^ j;
        if (y > x) {
          const float u = sW[x], v = sW[y];
          const bool asc = (x & k) == 0;
          if ((u > v) == asc) {
            sW[x] = v;
            sW[y] = u;
          }
        }
      }
      __syncthreads();
    }
  }
  const int b = bh / a.Hq, h = bh % a.Hq;
  for (int kk = tid; kk < a.n_budgets; kk += 256) {
    const int kb = a.budgets[kk];
    a.kth[(((long long)kk * a.B + b) * a.Hq + h) * a.nqb + i] =
        n_cand >= kb ? sW[P - kb] : kNegInf;
  }
}

// ---------------------------------------------------------------------------------------------
// Block means for mean correction ("FlashPrefill V2", mean correction): the mean key and mean
// value of every whole gate block of every (batch, KV head). The mean key goes out as two bf16
// parts, hi = bf16(mean) and lo = bf16(mean - hi), so that the stand-in's logit keeps about 16
// mantissa bits through the bf16 MFMA; the mean value as one bf16 row. One wave per block:
// lane l sums dims 8 (l % LPR) .. + 7 over rows l / LPR, l / LPR + RPI, .. in fp32 (16-byte
// loads, RPI rows per load), then the lanes of equal l % LPR add up their sums. A streaming
// read of K and V once: HBM-bound.
// ---------------------------------------------------------------------------------------------
template <int D, bool PAGED>
__global__ __launch_bounds__(256) void block_mean_kernel(PrefillArgs a) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RPI = 64 / LPR;       // rows per load
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int per = (a.mean_blocks + 3) / 4;    // workgroups per (batch, KV head)
  const int bg = blockIdx.x / per;
  const int J = (blockIdx.x % per) * 4 + w;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const Seq sq = seq_of(a, b);
  const int bkeys = a.kpb * kBlockK;
  if (J >= min(sq.Nk / bkeys, a.mean_blocks)) return;   // past this sequence's whole blocks
  const long long kst = a.ks[1], vst = a.vs[1];
  const __bf16* const Kb = static_cast<const __bf16*>(a.k) + sq.k + g * a.ks[2];
  const __bf16* const Vb = static_cast<const __bf16*>(a.v) + sq.v + g * a.vs[2];
  const int col = (lane % LPR) * 8;
  float ksum[8], vsum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) ksum[e] = vsum[e] = 0.f;
#pragma unroll 4
  for (int r = lane / LPR; r < bkeys; r += RPI) {
    const int key = J * bkeys + r;
    const int t = key / kBlockK, rt = key % kBlockK;
    const bf16x8 kx = *reinterpret_cast<const bf16x8*>(
        Kb + tile_offset<PAGED>(a, b, t, kst, a.ks[0]) + rt * kst + col);
    const bf16x8 vx = *reinterpret_cast<const bf16x8*>(
        Vb + tile_offset<PAGED>(a, b, t, vst, a.vs[0]) + rt * vst + col);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ksum[e] += (float)kx[e];
      vsum[e] += (float)vx[e];
    }
  }
#pragma unroll
  for (int x = LPR; x < 64; x <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ksum[e] += __shfl_xor(ksum[e], x);
      vsum[e] += __shfl_xor(vsum[e], x);
    }
  if (lane < LPR) {
    const float inv = 1.f / (float)bkeys;    // a power of two: exact
    bf16x8 hi, lo, vm;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float mk = ksum[e] * inv;
      hi[e] = (__bf16)mk;
      lo[e] = (__bf16)(mk - (float)hi[e]);
      vm[e] = (__bf16)(vsum[e] * inv);
    }
    const long long o = (((long long)b * a.Hkv + g) * a.mean_blocks + J) * D + col;
    *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(a.kbar_hi) + o) = hi;
    *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(a.kbar_lo) + o) = lo;
    *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(a.vbar) + o) = vm;
  }
}

// How many of the lowest query blocks a ticket-ordered softmax launch takes last, heaviest
// first across all KV heads (the blocks above go KV head by KV head). In KV-head order the
// last KV head's longest unit, about nqb key tiles per 64 query rows, starts near the end; the
// blocks below the cut, taken afterwards, must hold at least that much work per resident
// workgroup to keep the others busy meanwhile. Causal units at block i hold about i + 1 tiles
// per 64 rows, so the blocks below `cut` hold units * cut^2 / 2, i.e. units * cut^2 /
// (2 * resident) per workgroup: cut = sqrt(2 * resident * nqb / units). (The mask walk's units
// are shorter than causal ones, so the cut suits it too.)
inline int tail_query_blocks(int nqb, int units, int resident) {
  const double cut = ceil(sqrt(2.0 * resident * nqb / (double)units));
  return (int)fmin((double)nqb, cut);
}

template <int D, int BQ, int NW, bool PAGED>
hipError_t launch_prefill_paged(const PrefillArgs& a, int gate, hipStream_t stream) {
  const int units = a.units * a.nqb;
  // one workgroup per unit; with a ticket counter, as many as stay resident at once, each
  // taking units in turn: then in the order the workgroups start, one KV head at a time on
  // every XCD (its K/V stays in the last-level cache; a fixed KV-head-to-XCD assignment would
  // not hold, as any workgroup may take any unit), the lowest query blocks last, heaviest first
  // across all KV heads
  constexpr int HPW = NW / (BQ / kRows);
  auto go = [&](void (*kernel)(PrefillArgs), int loop) {
    if (loop == kTicketAlways && !a.ticket) return hipErrorInvalidValue;   // the mask walk
    PrefillArgs k = a;
    int n = units;
    if (loop != kOnePerUnit && a.ticket) {
      n = min(units, resident_workgroups(reinterpret_cast<const void*>(kernel), NW * 64, units));
      k.xcd_map = -1;
      k.tail_blocks = tail_query_blocks(a.nqb, a.units, n);
    } else {
      k.ticket = nullptr;
    }
    hipLaunchKernelGGL(kernel, dim3(n), dim3(NW * 64), 0, stream, k);
    return hipGetLastError();
  };
  switch (gate) {
    case kDense:
      return go(prefill_kernel<D, BQ, NW, kDense, PAGED>, kUnitLoop<kDense, HPW>);
    case kAbsolute:
    case kAbsVote:
      if constexpr (NW == BQ / kRows) {   // one head per workgroup
        if (gate == kAbsolute && a.kbar_hi)
          return go(prefill_kernel<D, BQ, NW, kAbsolute, PAGED, true>,
                    kUnitLoop<kAbsolute, HPW>);
        if (gate == kAbsolute)
          return go(prefill_kernel<D, BQ, NW, kAbsolute, PAGED>, kUnitLoop<kAbsolute, HPW>);
        return go(prefill_kernel<D, BQ, NW, kAbsVote, PAGED>, kUnitLoop<kAbsVote, HPW>);
      }
      return hipErrorInvalidConfiguration;
    default:
      return go(prefill_kernel<D, BQ, NW, kRelative, PAGED>, kUnitLoop<kRelative, HPW>);
  }
}

template <int D, int BQ, int NW>
hipError_t launch_calib_wg(const CalibArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((calibrate_kernel<D, BQ, NW>), dim3(a.units * a.nqb), dim3(NW * 64), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, int BQ>
hipError_t launch_calib_nw(const CalibArgs& a, int nw, hipStream_t stream) {
  switch (nw) {
    case 8: return launch_calib_wg<D, BQ, 8>(a, stream);
    case 4: return launch_calib_wg<D, BQ, 4>(a, stream);
    default: return launch_calib_wg<D, BQ, BQ / kRows>(a, stream);
  }
}

template <int D, int BQ>
hipError_t launch_sweep_hpw(const PrefillArgs& a, int hpw, hipStream_t stream) {
  constexpr int WPH = BQ / 64;
  const int units = a.units * a.nqb;
  // one workgroup per unit; with a ticket counter, as many as stay resident at once
  auto go = [&](void (*kernel)(PrefillArgs), int block) {
    const int n = a.ticket ? min(units, resident_workgroups(reinterpret_cast<const void*>(kernel),
                                                            block, units))
                           : units;
    hipLaunchKernelGGL(kernel, dim3(n), dim3(block), 0, stream, a);
    return hipGetLastError();
  };
  const bool paged = a.pages != nullptr;
  if (hpw == 2)
    return paged ? go(gate_sweep_kernel<D, BQ, 2, true>, WPH * 128)
                 : go(gate_sweep_kernel<D, BQ, 2, false>, WPH * 128);
  return paged ? go(gate_sweep_kernel<D, BQ, 1, true>, WPH * 64)
               : go(gate_sweep_kernel<D, BQ, 1, false>, WPH * 64);
}

}  // namespace

// Per (head dimension, query tile, K/V layout): the prefill kernel for any workgroup width and
// gate, the calibration kernel and the gate sweep. Each is instantiated explicitly by one
// translation unit.
// Waves per workgroup of the prefill kernel: BQ / 32 waves per head times 1 or 2 heads
// (BQ = 128: 4 waves; BQ = 64: 2 or 4 waves).
template <int D, int BQ, bool PAGED>
hipError_t launch_prefill_tile(const PrefillArgs& a, int nw, int gate, hipStream_t stream) {
  switch (nw) {
    case 4: return launch_prefill_paged<D, BQ, 4, PAGED>(a, gate, stream);
    default: return launch_prefill_paged<D, BQ, BQ / kRows, PAGED>(a, gate, stream);
  }
}

template <int D, int BQ>
hipError_t launch_calibrate_tile(const CalibArgs& a, int nw, hipStream_t stream) {
  return launch_calib_nw<D, BQ>(a, nw, stream);
}

inline hipError_t launch_kth_select_impl(const CalibArgs& a, const float* maxima, int block_q,
                                         hipStream_t stream) {
  hipLaunchKernelGGL(kth_select_kernel, dim3(a.B * a.Hq * a.nqb), dim3(256), 0, stream, a,
                     maxima, block_q);
  return hipGetLastError();
}

template <int D, int BQ>
hipError_t launch_sweep_tile(const PrefillArgs& a, int hpw, hipStream_t stream) {
  return launch_sweep_hpw<D, BQ>(a, hpw, stream);
}

template <int D, int BQ>
hipError_t launch_sweep_fp8_tile(const PrefillArgs& a, int hpw, hipStream_t stream) {
  constexpr int WPH = BQ / 64;
  const dim3 grid(a.units * a.nqb);
  if (hpw == 4)
    hipLaunchKernelGGL((gate_sweep_fp8_kernel<D, BQ, 4>), grid, dim3(WPH * 256), 0, stream, a);
  else if (hpw == 2)
    hipLaunchKernelGGL((gate_sweep_fp8_kernel<D, BQ, 2>), grid, dim3(WPH * 128), 0, stream, a);
  else
    hipLaunchKernelGGL((gate_sweep_fp8_kernel<D, BQ, 1>), grid, dim3(WPH * 64), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool PAGED>
hipError_t launch_quant_tile(const PrefillArgs& a, hipStream_t stream) {
  constexpr int RPB = 4 * 64 / (D / 8);
  const int per = (a.q8_rows * a.Hq + RPB - 1) / RPB;
  hipLaunchKernelGGL((quant_q_kernel<D>), dim3(a.B * per), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((quant_k_kernel<D, PAGED>), dim3(a.B * a.Hkv * a.k8_tiles), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, bool PAGED>
hipError_t launch_means_tile(const PrefillArgs& a, hipStream_t stream) {
  const int per = (a.mean_blocks + 3) / 4;
  hipLaunchKernelGGL((block_mean_kernel<D, PAGED>), dim3(a.B * a.Hkv * per), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace bsfa
