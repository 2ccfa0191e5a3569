// Internal interface between the C ABI (bsfa_api.cpp) and the HIP kernels (device code in
// bsfa_device.h, instantiated by the bsfa_*.hip units).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsfa {

constexpr int kBlockK = 64;          // key tile width (gate tile columns)
constexpr int kCalibMaxKeyBlocks = 4096;

// Prefill kernel instantiations: the public gate modes, plus the absolute gate decided inside
// the softmax loop (kAbsVote, used when no keep masks are given).
enum Gate : int { kDense = 0, kAbsolute = 1, kRelative = 2, kAbsVote = 3 };

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const float* thr;                // threshold slice [Hq][t_len] (ABSOLUTE) or nullptr
  int32_t* kept_counts;            // [B][Hq][nqb] or nullptr
  unsigned long long* kept_total;  // scalar or nullptr
  float* dbg;                      // [B][Hq][nqb][nkb] or nullptr
  long long qs[3], ks[3], vs[3], os[3];
  int B, N, Hq, Hkv, G, nqb, nkb, t_len;
  int Nk, P;                       // key tokens and the prefix before the query rows (Nk - N)
  // variable-length batches: token offsets of each sequence's queries and keys [B + 1] (the
  // sequences packed along the token axis; N, Nk are then the longest), or nullptr
  const int* cu_q;
  const int* cu_k;
  // paged K / V (with cu_q): K and V live in pages of page_tiles * 64 tokens; sequence b's key
  // tokens are kv_lens[b], its page j is pages[b * pages_stride + j]; ks[0] / vs[0] are the
  // page strides. nullptr: contiguous sequences.
  const int* pages;
  const int* kv_lens;
  int pages_stride, page_tiles;
  int units;                       // B * Hkv * (G / heads per workgroup)
  int xcd_map;                     // 1: each XCD serves fixed units (whole KV heads);
                                   // -1: KV-head-major order over all XCDs (the
                                   // query blocks below tail_blocks excepted)
  int xcd_rot;                     // with xcd_map: turn that assignment every xcd_rot query
                                   // blocks (0: never)
  int tail_blocks;                 // with xcd_map = -1: query blocks below this come last,
                                   // heaviest first, every KV head's units of a block together
  unsigned* ticket;                // counters, zero at the launch, from which the workgroups
                                   // resident at once take units in turn until all are taken
                                   // (the gate sweep with xcd_map = 1: one per XCD queue);
                                   // nullptr: one workgroup per unit
  float scale;                     // softmax scale applied to fp32 scores
  float c_log2;                    // scale * log2(e)
  float log_lambda;                // RELATIVE threshold
  int out_fp32;
  // ABSOLUTE: keep bitmasks from the gate sweep, [B][Hq][nqb][mask_words] (bit j of word
  // j / 64: off-diagonal tile j kept), or nullptr to find them inside the prefill kernel
  unsigned long long* keep_mask;
  int mask_words;
  int full_masks;                  // gate sweep: write every mask word of every (b, h, i)
  // 64-key tiles per gate block (block_k / 64: 1, or 2 for 128-key blocks). Loads and loop
  // iterations stay at 64 keys; decisions, kept counts and the statistic dump are per block,
  // and a kept block sets the mask bits of all its tiles. nkb counts gate blocks.
  int kpb;
  // Mean correction (ABSOLUTE walk): the mean key of every whole gate block as two bf16 parts
  // (kbar_hi = bf16(mean), kbar_lo = bf16(mean - kbar_hi)) and its mean value, each
  // [B][Hkv][mean_blocks][D]; kbar_hi == nullptr: no correction. mean_bias = ln(block keys) /
  // scale, the stand-in logit's shift in raw score units.
  void* kbar_hi;
  void* kbar_lo;
  void* vbar;
  int mean_blocks;
  float mean_bias;
  // FP8 gate scores (ABSOLUTE sweep): E4M3 copies of Q [B][q8_rows][Hq][D] and K
  // [B][k8_rows][Hkv][D] with fp32 scales per (b, h, row) [B][Hq][q8_rows] and per (b, g,
  // 64-key tile) [B][Hkv][k8_tiles]; q8 == nullptr: bf16 scores.
  void* q8;
  float* q8_scale;
  void* k8;
  float* k8_scale;
  int q8_rows, k8_rows, k8_tiles;
};

struct CalibArgs {
  const void* q;
  const void* k;
  long long qs[3], ks[3];
  int B, N, Hq, Hkv, G, nqb, nkb;
  int units, xcd_map, xcd_rot;
  float scale;
  int kpb;                         // 64-key tiles per gate block
  int n_budgets;
  int budgets[16];
  float* kth;                      // [n_budgets][B][Hq][nqb]
};

// Largest K / V token stride (elements): 64 rows of it stay below 4 GB, so tile offsets fit in
// 32 bits.
constexpr int64_t kMaxTokenStride = int64_t(1) << 25;

constexpr int kRowsPerWave = 32;

// Workgroup shape: waves of kRowsPerWave query rows; a workgroup holds the waves of 1, 2 or 4
// query heads of one KV group for one block of block_q rows (at most 8 waves). Returns the
// number of waves; heads per workgroup = waves / (block_q / kRowsPerWave).
int waves_per_workgroup(int block_q, int group);

// The prefill kernel's workgroup: as above, except that the absolute gate runs one head per
// workgroup (its keep decisions are made per head before the softmax pass).
int prefill_waves_per_workgroup(int block_q, int group, int gate);

// Workgroups of `kernel` (block threads, static LDS only) that the current device holds at
// once: its CUs times the workgroups per CU that the kernel's registers and LDS allow. Cached
// per (device, kernel); `fallback` if the runtime cannot tell.
int resident_workgroups(const void* kernel, int block, int fallback);

// Largest number of off-diagonal key tiles per query block under the absolute gate (the
// keep bitmask lives in LDS): 32768 tiles of 64 keys.
constexpr int kMaxGateTiles = 32768;

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int block_q, int gate,
                          hipStream_t stream);
hipError_t launch_calibrate(const CalibArgs& a, int head_dim, int block_q, hipStream_t stream);
// k-th highest per (budget, b, h, i) from a dump of the off-diagonal gate-block maxima
// (fp32 [B][Hq][nqb][nkb]); uses a.B, Hq, nqb, nkb, kpb, budgets, n_budgets, kth.
hipError_t launch_kth_select(const CalibArgs& a, const float* maxima, int block_q,
                             hipStream_t stream);
// The gate sweep for the absolute gate: fills a.keep_mask (and the off-diagonal entries of
// a.dbg). a.units must describe launch_gate_sweep's own workgroups (gate_sweep_heads()).
hipError_t launch_gate_sweep(const PrefillArgs& a, int head_dim, int block_q, hipStream_t stream);
// Heads per workgroup of the gate sweep (bf16 or FP8 scores).
int gate_sweep_heads(int block_q, int group, bool fp8);
hipError_t launch_zero_u64(unsigned long long* p, hipStream_t stream);
// n (1..64) consecutive 32-bit words set to zero by a kernel (no memset node in a graph)
hipError_t launch_zero_words(unsigned* p, int n, hipStream_t stream);
// The ticket counters at the end of the absolute gate's workspace: the gate sweep's, one per
// XCD queue (kSweepTickets), then the walk's.
constexpr int kSweepTickets = 8;
constexpr int kTickets = kSweepTickets + 1;
// The MFMA rate probe: workgroups x 4 waves, each 4 * iters bf16 32x32x16 MFMAs; sink holds
// workgroups * 256 floats.
hipError_t launch_mfma_rate(int workgroups, int iters, float* sink, hipStream_t stream);

// Block means for mean correction: fills a.kbar_hi, a.kbar_lo and a.vbar for every whole gate
// block of every (batch, KV head) (a.mean_blocks per sequence at most).
hipError_t launch_block_means(const PrefillArgs& a, int head_dim, hipStream_t stream);
// FP8 gate: fills a.q8 / a.q8_scale and a.k8 / a.k8_scale from Q and K.
hipError_t launch_quantize_qk(const PrefillArgs& a, int head_dim, hipStream_t stream);

// Launchers of one (head dimension D, query tile BQ[, paged K/V]) instantiation; each is defined
// in its own translation unit. nw = waves per workgroup, hpw = heads per sweep workgroup.
template <int D, int BQ, bool PAGED>
hipError_t launch_prefill_tile(const PrefillArgs& a, int nw, int gate, hipStream_t stream);
template <int D, int BQ>
hipError_t launch_calibrate_tile(const CalibArgs& a, int nw, hipStream_t stream);
template <int D, int BQ>
hipError_t launch_sweep_tile(const PrefillArgs& a, int hpw, hipStream_t stream);
template <int D, bool PAGED>
hipError_t launch_means_tile(const PrefillArgs& a, hipStream_t stream);
template <int D, bool PAGED>
hipError_t launch_quant_tile(const PrefillArgs& a, hipStream_t stream);
template <int D, int BQ>
hipError_t launch_sweep_fp8_tile(const PrefillArgs& a, int hpw, hipStream_t stream);

}  // namespace bsfa
