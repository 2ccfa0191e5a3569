// C ABI of libbsfa.so (declared in include/bsfa.h): host-side validation and dispatch.
//
// Every check runs on the host before anything is enqueued, so an error status means no GPU
// work was started and no output was touched. Nothing here synchronises or allocates.
#include "bsfa.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "bsfa_internal.h"

namespace {

thread_local char g_last_error[512] = "";

bsfa_status fail(bsfa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

bsfa_status ok() {
  g_last_error[0] = '\0';
  return BSFA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

float effective_scale(const bsfa_problem* p) {
  return p->softmax_scale > 0.f ? p->softmax_scale : 1.f / sqrtf((float)p->head_dim);
}

// Shape, tile, dtype and stride checks shared by both entry points.
bsfa_status check_problem(const bsfa_problem* p, bool need_v_o) {
  if (!p) return fail(BSFA_ERR_ARG, "problem is NULL");
  if (p->batch < 0 || p->seqlen < 0)
    return fail(BSFA_ERR_ARG, "batch (%d) and seqlen (%d) must be >= 0", p->batch, p->seqlen);
  if (p->heads_q < 1 || p->heads_kv < 1)
    return fail(BSFA_ERR_ARG, "heads_q (%d) and heads_kv (%d) must be >= 1", p->heads_q,
                p->heads_kv);
  if (p->kv_seqlen != 0 && p->kv_seqlen < p->seqlen)
    return fail(BSFA_ERR_ARG, "kv_seqlen (%d) must be 0 or >= seqlen (%d)", p->kv_seqlen,
                p->seqlen);
  if (p->heads_q % p->heads_kv != 0)
    return fail(BSFA_ERR_SHAPE, "heads_q (%d) is not a multiple of heads_kv (%d)", p->heads_q,
                p->heads_kv);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(BSFA_ERR_SHAPE, "head_dim %d not supported (64 or 128)", p->head_dim);
  const bool tile_ok = (p->block_k == bsfa::kBlockK && (p->block_q == 64 || p->block_q == 128)) ||
                       (p->block_k == 2 * bsfa::kBlockK && p->block_q == 128);
  if (!tile_ok)
    return fail(BSFA_ERR_SHAPE, "tile %dx%d not supported (64x64, 128x64 or 128x128)",
                p->block_q, p->block_k);
  if (!(p->softmax_scale >= 0.f) || isinf(p->softmax_scale))
    return fail(BSFA_ERR_ARG, "softmax_scale must be finite and >= 0");
  if (p->in_dtype != BSFA_BF16)
    return fail(BSFA_ERR_DTYPE, "in_dtype %d not supported (bf16 only)", p->in_dtype);
  if (need_v_o && p->out_dtype != BSFA_BF16 && p->out_dtype != BSFA_FP32)
    return fail(BSFA_ERR_DTYPE, "out_dtype %d not supported", p->out_dtype);
  const int64_t* strides[4] = {p->q_stride, p->k_stride, p->v_stride, p->o_stride};
  const char* names[4] = {"q", "k", "v", "o"};
  const int n_checked = need_v_o ? 4 : 2;
  for (int t = 0; t < n_checked; ++t) {
    const int64_t unit = (t == 3 && p->out_dtype == BSFA_FP32) ? 4 : 8;  // elements per 16 B
    for (int a = 0; a < 3; ++a) {
      if (strides[t][a] < 0)
        return fail(BSFA_ERR_ARG, "%s_stride[%d] is negative", names[t], a);
      if (strides[t][a] % unit != 0)
        return fail(BSFA_ERR_ALIGN, "%s_stride[%d] = %lld breaks 16-byte row alignment",
                    names[t], a, (long long)strides[t][a]);
    }
  }
  if (p->k_stride[1] > bsfa::kMaxTokenStride || (need_v_o && p->v_stride[1] > bsfa::kMaxTokenStride))
    return fail(BSFA_ERR_UNSUPPORTED, "K/V token stride above %lld elements",
                (long long)bsfa::kMaxTokenStride);
  return BSFA_OK;
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Key tokens: the query rows are the last seqlen of kv_seqlen positions (0: a whole prefill).
int key_len(const bsfa_problem* p) { return p->kv_seqlen > 0 ? p->kv_seqlen : p->seqlen; }

// The threshold table against the problem: present, aligned, bound to the same heads, tile,
// head_dim and scale, and the budget slice in range.
bsfa_status check_table(const bsfa_problem* p, const bsfa_table* table, int32_t budget_slice) {
  const float scale = effective_scale(p);
  if (!table) return fail(BSFA_ERR_TABLE, "ABSOLUTE gate needs a threshold table");
  if (!table->T) return fail(BSFA_ERR_TABLE, "table->T is NULL");
  if ((reinterpret_cast<uintptr_t>(table->T) & 3u) != 0)
    return fail(BSFA_ERR_ALIGN, "table->T is not 4-byte aligned");
  if (table->n_budgets < 1 || table->t_len < 1)
    return fail(BSFA_ERR_TABLE, "table has n_budgets %d, t_len %d", table->n_budgets,
                table->t_len);
  if (budget_slice < 0 || budget_slice >= table->n_budgets)
    return fail(BSFA_ERR_TABLE, "budget_slice %d outside [0, %d)", budget_slice,
                table->n_budgets);
  if (table->heads_q != p->heads_q || table->block_q != p->block_q ||
      table->block_k != p->block_k || table->head_dim != p->head_dim)
    return fail(BSFA_ERR_TABLE,
                "table calibrated for Hq=%d tile %dx%d d=%d, problem has Hq=%d tile %dx%d d=%d",
                table->heads_q, table->block_q, table->block_k, table->head_dim, p->heads_q,
                p->block_q, p->block_k, p->head_dim);
  if (!(fabsf(table->softmax_scale - scale) <= 1e-6f * scale))
    return fail(BSFA_ERR_TABLE, "table softmax_scale %g differs from the problem's %g",
                (double)table->softmax_scale, (double)scale);
  return BSFA_OK;
}

// Whether one launch (decisions inside the softmax loop) beats two (gate sweep, then a walk
// over the kept tiles) for this call. Only when the table records the slice's budget k: then
// (a) if the share of off-diagonal gate blocks the budget keeps if it held exactly,
// sum_i min(n_off(i), k) / sum_i n_off(i), is above 1/2 (the budget is a target count of kept
// blocks per query block, "Block Sparse Flash Attention", Method > Key Designs 1): with most
// blocks kept, a second pass over them costs more than deciding inside the softmax loop; or
// (b) if the call has fewer than 2^16 off-diagonal tiles in all (B * Hq * sum_i n_off(i)):
// then the second launch's fixed costs outweigh the work it saves. Unknown budgets (no array,
// k <= 0) keep two launches. For a variable-length batch the longest sequence stands for all.
bool one_launch_pays(const bsfa_problem* p, const bsfa_table* table, int32_t budget_slice) {
  if (!table || !table->budgets) return false;
  const long long k = table->budgets[budget_slice];
  if (k <= 0) return false;
  const long long pre = key_len(p) - p->seqlen;
  long long kept = 0, all = 0;
  for (int i = 0; i < ceil_div(p->seqlen, p->block_q); ++i) {
    const long long n_off = (pre + (long long)i * p->block_q) / p->block_k;
    kept += n_off < k ? n_off : k;
    all += n_off;
  }
  if (all > 0 && 2 * kept > all) return true;
  return (long long)p->batch * p->heads_q * all < (1ll << 16);
}

// Kernel arguments common to the prefill kernel and the gate sweep.
bsfa::PrefillArgs base_args(const bsfa_problem* p, const void* Q, const void* K, const void* V,
                            const bsfa_table* table, int32_t budget_slice, int32_t gate_mode) {
  bsfa::PrefillArgs a;
  memset(&a, 0, sizeof(a));
  const float scale = effective_scale(p);
  a.q = Q;
  a.k = K;
  a.v = V;
  a.thr = gate_mode == BSFA_GATE_ABSOLUTE
              ? table->T + (long long)budget_slice * table->heads_q * table->t_len
              : nullptr;
  a.t_len = gate_mode == BSFA_GATE_ABSOLUTE ? table->t_len : 1;
  for (int t = 0; t < 3; ++t) {
    a.qs[t] = p->q_stride[t];
    a.ks[t] = p->k_stride[t];
    a.vs[t] = p->v_stride[t];
    a.os[t] = p->o_stride[t];
  }
  a.B = p->batch;
  a.N = p->seqlen;
  a.Nk = key_len(p);
  a.P = a.Nk - a.N;
  a.Hq = p->heads_q;
  a.Hkv = p->heads_kv;
  a.G = p->heads_q / p->heads_kv;
  a.nqb = ceil_div(p->seqlen, p->block_q);
  a.nkb = ceil_div(a.Nk, p->block_k);
  a.kpb = p->block_k / bsfa::kBlockK;
  a.scale = scale;
  a.c_log2 = scale * 1.4426950408889634f;
  a.mask_words = ceil_div(ceil_div(a.Nk, bsfa::kBlockK), 64);
  return a;
}

// The absolute gate's workspace: the keep bitmasks (one bit per 64-key tile; a gate block of
// 128 keys sets two); then, every part on a 256-byte boundary, for an FP8 gate the E4M3 copies
// of Q and K and their scales, for mean correction the block means of K (bf16 high and low
// parts) and of V, [B][Hkv][mean_blocks][d] each, and last the walk's ticket counter.
struct WorkspaceLayout {
  uint64_t mask_bytes;
  int q8_rows, k8_rows, k8_tiles;
  uint64_t q8, q8_scale, k8, k8_scale, fp8_end;   // byte offsets
  int mean_blocks;
  uint64_t kbar_hi, kbar_lo, vbar, means_end;     // byte offsets
  uint64_t ticket, total;                         // byte offset of the counter; the whole size
};

uint64_t align256(uint64_t x) { return (x + 255u) & ~uint64_t(255); }

// DENSE and RELATIVE: the workspace holds only the softmax launch's ticket counter.
constexpr uint64_t kTicketBytes = 256;

WorkspaceLayout workspace_layout(const bsfa_problem* p) {
  WorkspaceLayout l;
  const uint64_t nqb = ceil_div(p->seqlen, p->block_q);
  const uint64_t words = ceil_div(ceil_div(key_len(p), bsfa::kBlockK), 64);
  l.mask_bytes = (uint64_t)p->batch * p->heads_q * nqb * words * 8u;
  const bool fp8 = p->gate_dtype == BSFA_FP8_E4M3;
  l.q8_rows = p->seqlen;
  l.k8_rows = key_len(p);
  l.k8_tiles = ceil_div(key_len(p), bsfa::kBlockK);
  const uint64_t B = p->batch, d = p->head_dim;
  l.q8 = align256(l.mask_bytes);
  l.q8_scale = l.q8 + (fp8 ? align256(B * l.q8_rows * p->heads_q * d) : 0);
  l.k8 = l.q8_scale + (fp8 ? align256(B * p->heads_q * l.q8_rows * 4u) : 0);
  l.k8_scale = l.k8 + (fp8 ? align256(B * l.k8_rows * p->heads_kv * d) : 0);
  l.fp8_end = l.k8_scale + (fp8 ? align256(B * p->heads_kv * l.k8_tiles * 4u) : 0);
  l.mean_blocks = key_len(p) / p->block_k;
  const uint64_t part = (uint64_t)p->batch * p->heads_kv * l.mean_blocks * p->head_dim * 2u;
  l.kbar_hi = l.fp8_end;
  l.kbar_lo = l.kbar_hi + align256(part);
  l.vbar = l.kbar_lo + align256(part);
  l.means_end = l.vbar + align256(part);
  l.ticket = align256(p->mean_correction ? l.means_end : fp8 ? l.fp8_end : l.mask_bytes);
  l.total = l.ticket + 256u;
  return l;
}

// FP8 gate: point `a` at the copies in the workspace and quantise Q and K into them.
hipError_t set_fp8(bsfa::PrefillArgs& a, const bsfa_problem* p, void* workspace, hipStream_t st) {
  const WorkspaceLayout l = workspace_layout(p);
  char* const ws = static_cast<char*>(workspace);
  a.q8 = ws + l.q8;
  a.q8_scale = reinterpret_cast<float*>(ws + l.q8_scale);
  a.k8 = ws + l.k8;
  a.k8_scale = reinterpret_cast<float*>(ws + l.k8_scale);
  a.q8_rows = l.q8_rows;
  a.k8_rows = l.k8_rows;
  a.k8_tiles = l.k8_tiles;
  return bsfa::launch_quantize_qk(a, p->head_dim, st);
}

// The gate sweep launch over `a` (keep_mask set): one workgroup per (b, head pair, i), or with
// a ticket counter (bf16 scores only) the resident workgroups taking those units in turn.
hipError_t launch_sweep(bsfa::PrefillArgs sw, const bsfa_problem* p, hipStream_t st) {
  const int shpw = bsfa::gate_sweep_heads(p->block_q, sw.G, sw.q8 != nullptr);
  sw.units = p->batch * p->heads_kv * (sw.G / shpw);
  if (sw.q8) sw.ticket = nullptr;
  // each XCD serves fixed KV heads (their K streams shared through its L2); with tickets it
  // takes its own units first and then helps the others. Unit counts that the XCDs cannot
  // share that way: with tickets one KV head at a time on every XCD
  sw.xcd_map = (sw.units % 8) == 0 ? 1 : sw.ticket ? -1 : 0;
  sw.xcd_rot = 0;
  return bsfa::launch_gate_sweep(sw, p->head_dim, p->block_q, st);
}

}  // namespace

extern "C" {

const char* bsfa_status_string(int32_t s) {
  switch (s) {
    case BSFA_OK: return "ok";
    case BSFA_ERR_ARG: return "invalid argument";
    case BSFA_ERR_SHAPE: return "unsupported or inconsistent shape";
    case BSFA_ERR_DTYPE: return "unsupported dtype";
    case BSFA_ERR_ALIGN: return "misaligned pointer or stride";
    case BSFA_ERR_TABLE: return "threshold table missing or inconsistent with the problem";
    case BSFA_ERR_UNSUPPORTED: return "unsupported request";
    case BSFA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* bsfa_last_error(void) { return g_last_error; }

int32_t bsfa_version(void) { return (3 << 16) | 3; }

uint64_t bsfa_prefill_workspace_bytes(const bsfa_problem* p, int32_t gate_mode) {
  if (!p || p->batch <= 0 || p->seqlen <= 0 || p->block_q <= 0 || p->block_k <= 0 ||
      p->heads_q <= 0)
    return 0;
  if (gate_mode == BSFA_GATE_DENSE || gate_mode == BSFA_GATE_RELATIVE) return kTicketBytes;
  return gate_mode == BSFA_GATE_ABSOLUTE ? workspace_layout(p).total : 0;
}

}  // extern "C"

namespace {

// Key layout of a variable-length batch: packed (cu_k) or paged (pages, kv_lens).
struct KeyLayout {
  const int32_t* cu_k = nullptr;
  const int32_t* pages = nullptr;
  const int32_t* kv_lens = nullptr;
  int32_t pages_stride = 0, page_size = 0;
};

// bsfa_prefill, bsfa_prefill_varlen and bsfa_prefill_paged: cu_q is NULL for a fixed-length
// batch.
bsfa_status prefill_impl(const bsfa_problem* p, const void* Q, const void* K, const void* V,
                         const int32_t* cu_q, const KeyLayout& kl, const bsfa_table* table,
                         int32_t budget_slice, int32_t gate_mode, float log_lambda, void* O,
                         int32_t* kept_counts, uint64_t* kept_total, float* debug_block_stat,
                         void* workspace, uint64_t workspace_bytes, void* stream,
                         bool validate_only = false) {
  const int32_t* cu_k = kl.cu_k;
  bsfa_status s = check_problem(p, true);
  if (s != BSFA_OK) return s;
  if (gate_mode != BSFA_GATE_DENSE && gate_mode != BSFA_GATE_ABSOLUTE &&
      gate_mode != BSFA_GATE_RELATIVE)
    return fail(BSFA_ERR_ARG, "gate_mode %d is not a bsfa_gate_mode", gate_mode);
  if (gate_mode == BSFA_GATE_RELATIVE && (isnan(log_lambda) || log_lambda == INFINITY))
    return fail(BSFA_ERR_ARG, "log_lambda must be finite or -INFINITY");
  if (gate_mode == BSFA_GATE_ABSOLUTE) {
    s = check_table(p, table, budget_slice);
    if (s != BSFA_OK) return s;
  }
  if (p->mean_correction != 0 && p->mean_correction != 1)
    return fail(BSFA_ERR_ARG, "mean_correction must be 0 or 1");
  // mean correction adds stand-ins for pruned blocks: after the absolute gate's sweep (the
  // relative gate decides from the running max, which a stand-in would move)
  const bool mean = p->mean_correction && gate_mode == BSFA_GATE_ABSOLUTE;
  if (p->mean_correction && gate_mode == BSFA_GATE_RELATIVE)
    return fail(BSFA_ERR_UNSUPPORTED, "mean correction is defined for the absolute gate");
  if (mean && !workspace)
    return fail(BSFA_ERR_UNSUPPORTED, "mean correction needs a workspace (the block means)");
  if (mean && (reinterpret_cast<uintptr_t>(workspace) & 15u))
    return fail(BSFA_ERR_ALIGN, "mean correction needs a 16-byte-aligned workspace");
  if (p->gate_dtype != BSFA_BF16 && p->gate_dtype != BSFA_FP8_E4M3)
    return fail(BSFA_ERR_DTYPE, "gate_dtype %d not supported (BF16 or FP8_E4M3)", p->gate_dtype);
  // FP8 gate scores: the absolute gate's sweep (the relative gate votes on the softmax's own
  // scores)
  const bool fp8 = p->gate_dtype == BSFA_FP8_E4M3 && gate_mode == BSFA_GATE_ABSOLUTE;
  if (p->gate_dtype == BSFA_FP8_E4M3 && gate_mode == BSFA_GATE_RELATIVE)
    return fail(BSFA_ERR_UNSUPPORTED, "FP8 gate scores are defined for the absolute gate");
  if (fp8 && !workspace)
    return fail(BSFA_ERR_UNSUPPORTED, "an FP8 gate needs a workspace (the FP8 copies)");
  if (fp8 && (reinterpret_cast<uintptr_t>(workspace) & 15u))
    return fail(BSFA_ERR_ALIGN, "an FP8 gate needs a 16-byte-aligned workspace");
  if (p->block_k != bsfa::kBlockK) {
    // 128-key gate blocks are decided by the gate sweep; a vote inside the softmax loop, which
    // walks 64-key tiles, is not built for them
    if (gate_mode == BSFA_GATE_RELATIVE)
      return fail(BSFA_ERR_UNSUPPORTED, "the relative gate takes 64-key blocks");
    if (gate_mode == BSFA_GATE_ABSOLUTE && !workspace)
      return fail(BSFA_ERR_UNSUPPORTED,
                  "128-key blocks under the absolute gate need a workspace (the gate sweep)");
    if (debug_block_stat)
      return fail(BSFA_ERR_UNSUPPORTED,
                  "128-key blocks: the block statistics come from bsfa_gate_masks");
  }
  const bool empty = p->batch == 0 || p->seqlen == 0;
  if (!empty) {
    if (cu_q && ((reinterpret_cast<uintptr_t>(cu_q) | reinterpret_cast<uintptr_t>(cu_k) |
                  reinterpret_cast<uintptr_t>(kl.pages) | reinterpret_cast<uintptr_t>(kl.kv_lens)) &
                 3u))
      return fail(BSFA_ERR_ALIGN, "cu_seqlens, block_table and kv_lens must be 4-byte aligned");
    if (!Q || !K || !V || !O) return fail(BSFA_ERR_ARG, "Q, K, V and O must be non-NULL");
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
      return fail(BSFA_ERR_ALIGN, "Q, K, V and O must be 16-byte aligned");
  }
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 7u))
    return fail(BSFA_ERR_ALIGN, "workspace is not 8-byte aligned");
  if ((kept_counts && (reinterpret_cast<uintptr_t>(kept_counts) & 3u)) ||
      (kept_total && (reinterpret_cast<uintptr_t>(kept_total) & 7u)) ||
      (debug_block_stat && (reinterpret_cast<uintptr_t>(debug_block_stat) & 3u)))
    return fail(BSFA_ERR_ALIGN, "kept_counts, kept_total or debug_block_stat misaligned");
  const int nqb = ceil_div(p->seqlen, p->block_q);
  const int nkb = ceil_div(key_len(p), bsfa::kBlockK);
  if ((long long)key_len(p) > (1ll << 30))
    return fail(BSFA_ERR_UNSUPPORTED, "kv_seqlen %d too large", key_len(p));
  if (gate_mode == BSFA_GATE_ABSOLUTE && nkb > bsfa::kMaxGateTiles)
    return fail(BSFA_ERR_UNSUPPORTED, "%d keys above the absolute-gate limit %d", key_len(p),
                bsfa::kMaxGateTiles * bsfa::kBlockK);
  if (gate_mode == BSFA_GATE_ABSOLUTE && (key_len(p) - p->seqlen) % p->block_q != 0)
    return fail(BSFA_ERR_SHAPE, "the absolute gate needs the prefix (%d keys) to be a multiple "
                "of block_q (%d): thresholds are indexed by absolute query block",
                key_len(p) - p->seqlen, p->block_q);
  if ((long long)p->batch * p->heads_q * nqb > 0x7fffffffll)
    return fail(BSFA_ERR_UNSUPPORTED, "grid too large");
  const uint64_t ws_need = bsfa_prefill_workspace_bytes(p, gate_mode);
  // the absolute gate with a workspace takes two launches unless one pays (the slice's
  // budget keeps most blocks, or the call is small); mean correction, FP8 scores and 128-key
  // blocks always take two
  const bool use_masks = gate_mode == BSFA_GATE_ABSOLUTE && workspace && !empty &&
                         (mean || fp8 || p->block_k != bsfa::kBlockK ||
                          !one_launch_pays(p, table, budget_slice));
  // one softmax launch (dense, the relative gate, the absolute gate decided in the loop): its
  // workgroups take their units from a counter in the workspace
  const bool use_ticket = !use_masks && workspace && !empty;
  if ((use_masks || use_ticket) && workspace_bytes < ws_need)
    return fail(BSFA_ERR_ARG, "workspace_bytes %llu below the required %llu",
                (unsigned long long)workspace_bytes, (unsigned long long)ws_need);

  if (validate_only) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (kept_total) {
    hipError_t e = bsfa::launch_zero_u64(reinterpret_cast<unsigned long long*>(kept_total), st);
    if (e != hipSuccess) return fail(BSFA_ERR_HIP, "zeroing kept_total: %s", hipGetErrorString(e));
  }
  if (empty) return ok();

  bsfa::PrefillArgs a = base_args(p, Q, K, V, table, budget_slice, gate_mode);
  a.o = O;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.pages = kl.pages;
  a.kv_lens = kl.kv_lens;
  a.pages_stride = kl.pages_stride;
  a.page_tiles = kl.page_size / bsfa::kBlockK;
  a.kept_counts = kept_counts;
  a.kept_total = reinterpret_cast<unsigned long long*>(kept_total);
  a.dbg = debug_block_stat;
  // the kernel instantiation: the absolute gate walks the sweep's masks, or without a
  // workspace decides every block inside the softmax loop
  const int kgate = gate_mode == BSFA_GATE_ABSOLUTE && !use_masks ? bsfa::kAbsVote : gate_mode;
  const int nw = bsfa::prefill_waves_per_workgroup(p->block_q, a.G, kgate);
  const int hpw = nw / (p->block_q / bsfa::kRowsPerWave);
  a.units = p->batch * p->heads_kv * (a.G / hpw);
  a.xcd_map = (a.units % 8) == 0;
  // the absolute gate decided in the loop: kept counts differ between heads (each has its own
  // thresholds), so the KV-head-to-XCD assignment turns every 16 query blocks (about as many
  // as are resident at once: 512 workgroups over 32 units at Bq = 128)
  if (kgate == bsfa::kAbsVote) a.xcd_rot = 16;
  a.log_lambda = log_lambda;
  a.out_fp32 = p->out_dtype == BSFA_FP32;
  // ABSOLUTE with a workspace: the gate sweep decides every block first (its own launch, so
  // that all workgroups stream K in step), then the prefill kernel runs over the kept ones
  if (use_masks) {
    a.keep_mask = static_cast<unsigned long long*>(workspace);
    if (fp8) {
      hipError_t e = set_fp8(a, p, workspace, st);
      if (e != hipSuccess) return fail(BSFA_ERR_HIP, "FP8 copies launch: %s", hipGetErrorString(e));
    }
    if (mean) {
      const WorkspaceLayout l = workspace_layout(p);
      char* const ws = static_cast<char*>(workspace);
      a.kbar_hi = ws + l.kbar_hi;
      a.kbar_lo = ws + l.kbar_lo;
      a.vbar = ws + l.vbar;
      a.mean_blocks = l.mean_blocks;
      a.mean_bias = logf((float)p->block_k) / a.scale;
      if (l.mean_blocks > 0) {
        hipError_t e = bsfa::launch_block_means(a, p->head_dim, st);
        if (e != hipSuccess)
          return fail(BSFA_ERR_HIP, "block means launch: %s", hipGetErrorString(e));
      }
    }
    // the ticket counters of the sweep (one per XCD queue) and of the walk, zeroed together
    unsigned* const tickets = reinterpret_cast<unsigned*>(static_cast<char*>(workspace) +
                                                          workspace_layout(p).ticket);
    hipError_t e = bsfa::launch_zero_words(tickets, bsfa::kTickets, st);
    if (e != hipSuccess) return fail(BSFA_ERR_HIP, "zeroing the tickets: %s", hipGetErrorString(e));
    a.ticket = tickets;
    e = launch_sweep(a, p, st);
    if (e != hipSuccess) return fail(BSFA_ERR_HIP, "gate sweep launch: %s", hipGetErrorString(e));
    // the walk over kept tiles: one KV head at a time on all XCDs (its K/V stays in the
    // last-level cache) but for the lowest query blocks, taken last, units in the order the
    // workgroups start (walk lengths differ, so a fixed assignment would load some XCDs more
    // than others)
    a.xcd_map = -1;
    a.ticket = tickets + bsfa::kSweepTickets;
  }
  if (use_ticket) {
    // the first word of the workspace, or of the absolute gate's ticket counters
    unsigned* const ticket = reinterpret_cast<unsigned*>(
        static_cast<char*>(workspace) +
        (gate_mode == BSFA_GATE_ABSOLUTE ? workspace_layout(p).ticket : 0));
    hipError_t e = bsfa::launch_zero_words(ticket, 1, st);
    if (e != hipSuccess) return fail(BSFA_ERR_HIP, "zeroing the ticket: %s", hipGetErrorString(e));
    a.ticket = ticket;
  }
  hipError_t e = bsfa::launch_prefill(a, p->head_dim, p->block_q, kgate, st);
  if (e != hipSuccess) return fail(BSFA_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return ok();
}

// ---- Static scratch for bsfa_prefill_noalloc ----
// The absolute gate's workspace (keep masks, block means) for callers that cannot allocate:
// one array per device, part of the library's code object, held until the process ends. In
// host code `scratch` names a host-side stand-in, not device memory: its device address is
// looked up once per device (with that device current) and only that address is used.
constexpr uint64_t kScratchBytes = uint64_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The current device's copy of the scratch array.
hipError_t scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace

extern "C" {

bsfa_status bsfa_prefill(const bsfa_problem* p, const void* Q, const void* K, const void* V,
                         const bsfa_table* table, int32_t budget_slice, int32_t gate_mode,
                         float log_lambda, void* O, int32_t* kept_counts, uint64_t* kept_total,
                         float* debug_block_stat, void* workspace, uint64_t workspace_bytes,
                         void* stream) {
  return prefill_impl(p, Q, K, V, nullptr, KeyLayout(), table, budget_slice, gate_mode,
                      log_lambda, O, kept_counts, kept_total, debug_block_stat, workspace,
                      workspace_bytes, stream);
}

bsfa_status bsfa_prefill_noalloc(const bsfa_problem* p, const void* Q, const void* K,
                                 const void* V, const bsfa_table* table, int32_t budget_slice,
                                 int32_t gate_mode, float log_lambda, void* O,
                                 int32_t* kept_counts, uint64_t* kept_total,
                                 float* debug_block_stat, void* stream) {
  bsfa_status s = check_problem(p, true);
  if (s != BSFA_OK) return s;
  // every gate takes the static scratch as its workspace
  const uint64_t need = bsfa_prefill_workspace_bytes(p, gate_mode);
  if (need > kScratchBytes)
    return fail(BSFA_ERR_UNSUPPORTED,
                "this call needs %llu bytes of workspace, above the %llu-byte static scratch of "
                "bsfa_prefill_noalloc (bsfa_prefill takes a caller workspace)",
                (unsigned long long)need, (unsigned long long)kScratchBytes);
  // every check first, against a stand-in with the scratch's size and alignment (never
  // dereferenced), so that an invalid call touches no device
  s = prefill_impl(p, Q, K, V, nullptr, KeyLayout(), table, budget_slice, gate_mode, log_lambda,
                   O, kept_counts, kept_total, debug_block_stat,
                   reinterpret_cast<void*>(uintptr_t(256)), kScratchBytes, stream, true);
  if (s != BSFA_OK) return s;
  void* ptr = nullptr;
  const hipError_t e = scratch_of_current_device(&ptr);
  if (e != hipSuccess || !ptr)
    return fail(BSFA_ERR_HIP, "device address of the static scratch: %s", hipGetErrorString(e));
  return prefill_impl(p, Q, K, V, nullptr, KeyLayout(), table, budget_slice, gate_mode,
                      log_lambda, O, kept_counts, kept_total, debug_block_stat, ptr,
                      kScratchBytes, stream);
}

bsfa_status bsfa_prefill_varlen(const bsfa_problem* p, const void* Q, const void* K,
                                const void* V, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_k, const bsfa_table* table,
                                int32_t budget_slice, int32_t gate_mode, float log_lambda, void* O,
                                int32_t* kept_counts, uint64_t* kept_total,
                                float* debug_block_stat, void* workspace,
                                uint64_t workspace_bytes, void* stream) {
  if (!p) return fail(BSFA_ERR_ARG, "problem is NULL");
  if (p->batch > 0 && p->seqlen > 0 && (!cu_seqlens_q || !cu_seqlens_k))
    return fail(BSFA_ERR_ARG, "cu_seqlens_q and cu_seqlens_k must be non-NULL");
  KeyLayout kl;
  kl.cu_k = cu_seqlens_k;
  return prefill_impl(p, Q, K, V, cu_seqlens_q, kl, table, budget_slice, gate_mode, log_lambda,
                      O, kept_counts, kept_total, debug_block_stat, workspace, workspace_bytes,
                      stream);
}

bsfa_status bsfa_prefill_paged(const bsfa_problem* p, const void* Q, const void* K_pages,
                               const void* V_pages, const int32_t* cu_seqlens_q,
                               const int32_t* kv_lens, const int32_t* block_table,
                               int32_t block_table_stride, int32_t page_size,
                               const bsfa_table* table, int32_t budget_slice, int32_t gate_mode,
                               float log_lambda, void* O, int32_t* kept_counts,
                               uint64_t* kept_total, float* debug_block_stat, void* workspace,
                               uint64_t workspace_bytes, void* stream) {
  if (!p) return fail(BSFA_ERR_ARG, "problem is NULL");
  if (page_size < bsfa::kBlockK || page_size % bsfa::kBlockK != 0)
    return fail(BSFA_ERR_SHAPE, "page_size %d must be a positive multiple of %d", page_size,
                bsfa::kBlockK);
  const int max_k = p->kv_seqlen > 0 ? p->kv_seqlen : p->seqlen;
  if (block_table_stride < ceil_div(max_k, page_size))
    return fail(BSFA_ERR_ARG, "block_table_stride %d below the pages of %d keys",
                block_table_stride, max_k);
  if (p->batch > 0 && p->seqlen > 0 && (!cu_seqlens_q || !kv_lens || !block_table))
    return fail(BSFA_ERR_ARG, "cu_seqlens_q, kv_lens and block_table must be non-NULL");
  KeyLayout kl;
  kl.pages = block_table;
  kl.kv_lens = kv_lens;
  kl.pages_stride = block_table_stride;
  kl.page_size = page_size;
  return prefill_impl(p, Q, K_pages, V_pages, cu_seqlens_q, kl, table, budget_slice, gate_mode,
                      log_lambda, O, kept_counts, kept_total, debug_block_stat, workspace,
                      workspace_bytes, stream);
}

bsfa_status bsfa_gate_masks(const bsfa_problem* p, const void* Q, const void* K,
                            const bsfa_table* table, int32_t budget_slice, uint64_t* keep_mask,
                            uint64_t mask_bytes, float* debug_block_stat, void* stream) {
  bsfa_status s = check_problem(p, false);
  if (s != BSFA_OK) return s;
  s = check_table(p, table, budget_slice);
  if (s != BSFA_OK) return s;
  const bool empty = p->batch == 0 || p->seqlen == 0;
  if (empty) return ok();
  if (!Q || !K || !keep_mask) return fail(BSFA_ERR_ARG, "Q, K and keep_mask must be non-NULL");
  if (!aligned16(Q) || !aligned16(K)) return fail(BSFA_ERR_ALIGN, "Q and K must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(keep_mask) & 7u)
    return fail(BSFA_ERR_ALIGN, "keep_mask is not 8-byte aligned");
  if (debug_block_stat && (reinterpret_cast<uintptr_t>(debug_block_stat) & 3u))
    return fail(BSFA_ERR_ALIGN, "debug_block_stat misaligned");
  const int nqb = ceil_div(p->seqlen, p->block_q);
  const int nkb = ceil_div(key_len(p), bsfa::kBlockK);
  if (nkb > bsfa::kMaxGateTiles)
    return fail(BSFA_ERR_UNSUPPORTED, "%d keys above the absolute-gate limit %d", key_len(p),
                bsfa::kMaxGateTiles * bsfa::kBlockK);
  if ((key_len(p) - p->seqlen) % p->block_q != 0)
    return fail(BSFA_ERR_SHAPE, "the absolute gate needs the prefix (%d keys) to be a multiple "
                "of block_q (%d): thresholds are indexed by absolute query block",
                key_len(p) - p->seqlen, p->block_q);
  if ((long long)p->batch * p->heads_q * nqb > 0x7fffffffll)
    return fail(BSFA_ERR_UNSUPPORTED, "grid too large");
  if (p->gate_dtype != BSFA_BF16 && p->gate_dtype != BSFA_FP8_E4M3)
    return fail(BSFA_ERR_DTYPE, "gate_dtype %d not supported (BF16 or FP8_E4M3)", p->gate_dtype);
  const bool fp8 = p->gate_dtype == BSFA_FP8_E4M3;
  // with an FP8 gate the buffer continues with the FP8 copies
  const uint64_t need = fp8 ? workspace_layout(p).fp8_end : workspace_layout(p).mask_bytes;
  if (mask_bytes < need)
    return fail(BSFA_ERR_ARG, "mask_bytes %llu below the required %llu",
                (unsigned long long)mask_bytes, (unsigned long long)need);
  if (fp8 && (reinterpret_cast<uintptr_t>(keep_mask) & 15u))
    return fail(BSFA_ERR_ALIGN, "an FP8 gate needs a 16-byte-aligned keep_mask buffer");
  bsfa::PrefillArgs a = base_args(p, Q, K, nullptr, table, budget_slice, BSFA_GATE_ABSOLUTE);
  a.keep_mask = reinterpret_cast<unsigned long long*>(keep_mask);
  a.dbg = debug_block_stat;
  a.full_masks = 1;
  if (fp8) {
    hipError_t e = set_fp8(a, p, keep_mask, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(BSFA_ERR_HIP, "FP8 copies launch: %s", hipGetErrorString(e));
  }
  // a buffer the size of bsfa_prefill's workspace: the bf16 sweep takes its units from the
  // workspace's ticket counter, as it does inside bsfa_prefill
  const WorkspaceLayout l = workspace_layout(p);
  if (!fp8 && mask_bytes >= l.total) {
    a.ticket = reinterpret_cast<unsigned*>(reinterpret_cast<char*>(keep_mask) + l.ticket);
    hipError_t e = bsfa::launch_zero_words(a.ticket, bsfa::kSweepTickets,
                                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(BSFA_ERR_HIP, "zeroing the ticket: %s", hipGetErrorString(e));
  }
  hipError_t e = launch_sweep(a, p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(BSFA_ERR_HIP, "gate sweep launch: %s", hipGetErrorString(e));
  return ok();
}

bsfa_status bsfa_mfma_rate_probe(int32_t workgroups, int32_t iters, float* sink, void* stream) {
  if (workgroups < 1 || iters < 1 || !sink)
    return fail(BSFA_ERR_ARG, "workgroups (%d) and iters (%d) must be >= 1, sink non-NULL",
                workgroups, iters);
  if (reinterpret_cast<uintptr_t>(sink) & 3u) return fail(BSFA_ERR_ALIGN, "sink misaligned");
  hipError_t e = bsfa::launch_mfma_rate(workgroups, iters, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(BSFA_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
  return ok();
}

uint64_t bsfa_calibrate_workspace_bytes(const bsfa_problem* p) {
  if (!p || p->gate_dtype != BSFA_FP8_E4M3 || p->batch <= 0 || p->seqlen <= 0 ||
      p->block_q <= 0 || p->block_k <= 0 || p->heads_q <= 0)
    return 0;
  const WorkspaceLayout l = workspace_layout(p);
  return align256(l.fp8_end) + (uint64_t)p->batch * p->heads_q * ceil_div(p->seqlen, p->block_q) *
                                   ceil_div(p->seqlen, p->block_k) * 4u;
}

bsfa_status bsfa_calibrate_blockmax(const bsfa_problem* p, const void* Q, const void* K,
                                    const int32_t* budgets_host, int32_t n_budgets,
                                    float* kth_out, void* workspace, uint64_t workspace_bytes,
                                    void* stream) {
  bsfa_status s = check_problem(p, false);
  if (s != BSFA_OK) return s;
  if (n_budgets < 1 || n_budgets > 16)
    return fail(BSFA_ERR_ARG, "n_budgets %d outside 1..16", n_budgets);
  if (!budgets_host) return fail(BSFA_ERR_ARG, "budgets_host is NULL");
  for (int t = 0; t < n_budgets; ++t)
    if (budgets_host[t] < 1) return fail(BSFA_ERR_ARG, "budget %d is < 1", budgets_host[t]);
  if (key_len(p) != p->seqlen)
    return fail(BSFA_ERR_UNSUPPORTED, "calibration takes whole sequences (kv_seqlen 0 or seqlen)");
  if (p->gate_dtype != BSFA_BF16 && p->gate_dtype != BSFA_FP8_E4M3)
    return fail(BSFA_ERR_DTYPE, "gate_dtype %d not supported (BF16 or FP8_E4M3)", p->gate_dtype);
  const bool fp8 = p->gate_dtype == BSFA_FP8_E4M3;
  const int nkb = ceil_div(p->seqlen, bsfa::kBlockK);   // 64-key tiles
  if (nkb > bsfa::kCalibMaxKeyBlocks)
    return fail(BSFA_ERR_UNSUPPORTED, "seqlen %d above the calibration limit %d", p->seqlen,
                bsfa::kCalibMaxKeyBlocks * bsfa::kBlockK);
  const bool empty = p->batch == 0 || p->seqlen == 0;
  if (empty) return ok();
  if (!Q || !K || !kth_out) return fail(BSFA_ERR_ARG, "Q, K and kth_out must be non-NULL");
  if (!aligned16(Q) || !aligned16(K)) return fail(BSFA_ERR_ALIGN, "Q and K must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(kth_out) & 3u) return fail(BSFA_ERR_ALIGN, "kth_out misaligned");
  const uint64_t ws_need = bsfa_calibrate_workspace_bytes(p);
  if (fp8 && !workspace)
    return fail(BSFA_ERR_ARG, "FP8 calibration needs a workspace of %llu bytes",
                (unsigned long long)ws_need);
  if (fp8 && (reinterpret_cast<uintptr_t>(workspace) & 15u))
    return fail(BSFA_ERR_ALIGN, "the workspace is not 16-byte aligned");
  if (fp8 && workspace_bytes < ws_need)
    return fail(BSFA_ERR_ARG, "workspace_bytes %llu below the required %llu",
                (unsigned long long)workspace_bytes, (unsigned long long)ws_need);

  bsfa::CalibArgs a;
  memset(&a, 0, sizeof(a));
  a.q = Q;
  a.k = K;
  for (int t = 0; t < 3; ++t) {
    a.qs[t] = p->q_stride[t];
    a.ks[t] = p->k_stride[t];
  }
  a.B = p->batch;
  a.N = p->seqlen;
  a.Hq = p->heads_q;
  a.Hkv = p->heads_kv;
  a.G = p->heads_q / p->heads_kv;
  a.nqb = ceil_div(p->seqlen, p->block_q);
  a.nkb = nkb;
  a.kpb = p->block_k / bsfa::kBlockK;
  const int nw = bsfa::waves_per_workgroup(p->block_q, a.G);
  const int hpw = nw / (p->block_q / bsfa::kRowsPerWave);
  a.units = p->batch * p->heads_kv * (a.G / hpw);
  a.xcd_map = (a.units % 8) == 0;
  a.scale = effective_scale(p);
  a.n_budgets = n_budgets;
  for (int t = 0; t < n_budgets; ++t) a.budgets[t] = budgets_host[t];
  a.kth = kth_out;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (fp8) {
    // the FP8 gate sweep without a table dumps every off-diagonal block maximum; then the
    // k-th highest of each (b, h, i)
    char* const ws = static_cast<char*>(workspace);
    float* const maxima = reinterpret_cast<float*>(ws + align256(workspace_layout(p).fp8_end));
    bsfa::PrefillArgs sw = base_args(p, Q, K, nullptr, nullptr, 0, BSFA_GATE_DENSE);
    sw.keep_mask = reinterpret_cast<unsigned long long*>(ws);
    sw.dbg = maxima;
    hipError_t e = set_fp8(sw, p, workspace, st);
    if (e == hipSuccess) e = launch_sweep(sw, p, st);
    if (e != hipSuccess) return fail(BSFA_ERR_HIP, "FP8 maxima launch: %s", hipGetErrorString(e));
    bsfa::CalibArgs ca = a;
    ca.nkb = sw.nkb;   // the dump's row length: gate blocks
    e = bsfa::launch_kth_select(ca, maxima, p->block_q, st);
    if (e != hipSuccess) return fail(BSFA_ERR_HIP, "k-th select launch: %s", hipGetErrorString(e));
    return ok();
  }
  hipError_t e = bsfa::launch_calibrate(a, p->head_dim, p->block_q, st);
  if (e != hipSuccess) return fail(BSFA_ERR_HIP, "calibration launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
