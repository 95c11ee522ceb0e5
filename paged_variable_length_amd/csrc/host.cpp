// Host-side parts of libpagedattn.so: error state, packing, the Dynamic Decomposer's task
// table, workspace sizing and the block-table debug check. No HIP calls in this file.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <vector>

#include "internal.h"

namespace pa {

static thread_local char g_err[512] = "";

int clear_error() {
  g_err[0] = '\0';
  return PA_OK;
}

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

}  // namespace pa

using pa::set_error;

extern "C" int pa_abi_version(void) { return PA_ABI_VERSION; }

extern "C" const char* pa_last_error(void) { return pa::g_err; }

// Packing into cumulative offsets (cann-recipes-infer page, section 2.3).
extern "C" int pa_pack_seqlens(const int32_t* lengths, int32_t n, int32_t* cu) {
  if (!cu || (n > 0 && !lengths)) return set_error(PA_ERR_NULL, "pa_pack_seqlens: NULL pointer");
  if (n < 0) return set_error(PA_ERR_INPUT, "pa_pack_seqlens: negative count %d", n);
  int64_t run = 0;
  cu[0] = 0;
  for (int32_t s = 0; s < n; ++s) {
    if (lengths[s] < 1)
      return set_error(PA_ERR_INPUT, "pa_pack_seqlens: length[%d] = %d < 1", s, lengths[s]);
    run += lengths[s];
    if (run > INT32_MAX) return set_error(PA_ERR_INPUT, "pa_pack_seqlens: total overflows int32");
    cu[s + 1] = static_cast<int32_t>(run);
  }
  return pa::clear_error();
}

namespace {

int check_params(const pa_params* p) {
  if (p->num_q_heads < 1 || p->num_kv_heads < 1 || p->num_q_heads % p->num_kv_heads)
    return set_error(PA_ERR_SHAPE, "query heads (%d) must be a positive multiple of kv heads (%d)",
                     p->num_q_heads, p->num_kv_heads);
  if (!pa::block_size_ok(p->block_size))
    return set_error(PA_ERR_BLOCK_SIZE, "block_size %d is not a power of two in [16, 256]",
                     p->block_size);
  if (p->dec_split < pa::kSplitQuantum || p->dec_split % pa::kSplitQuantum)
    return set_error(PA_ERR_SHAPE, "dec_split %d must be a positive multiple of %d", p->dec_split,
                     pa::kSplitQuantum);
  if (p->pf_q_tile < 1 || p->pf_q_tile > pa::kMaxQTile)
    return set_error(PA_ERR_SHAPE, "pf_q_tile %d must lie in [1, %d]", p->pf_q_tile,
                     pa::kMaxQTile);
  if (p->pf_kv_split < 0 || p->pf_kv_split % pa::kSplitQuantum)
    return set_error(PA_ERR_SHAPE, "pf_kv_split %d must be 0 or a positive multiple of %d",
                     p->pf_kv_split, pa::kSplitQuantum);
  if (p->num_workers < 1 || p->decode_weight < 1)
    return set_error(PA_ERR_SHAPE, "num_workers and decode_weight must be >= 1");
  if (p->verify_rows != 0 && (p->verify_rows < 2 || p->verify_rows > pa::kMaxGroup))
    return set_error(PA_ERR_SHAPE, "verify_rows %d must be 0 or lie in [2, %d]", p->verify_rows,
                     pa::kMaxGroup);
  if (p->shared_min < 0 || p->shared_min % pa::kSplitQuantum)
    return set_error(PA_ERR_SHAPE, "shared_min %d must be 0 or a positive multiple of %d",
                     p->shared_min, pa::kSplitQuantum);
  if (p->reserved != 0) return set_error(PA_ERR_SHAPE, "pa_params.reserved must be zero");
  return PA_OK;
}

// A sequence of ql > 1 rows runs as verify tasks (all its rows and the G query heads of one kv
// head in one task, as 16 score columns) when verify_rows allows it and G*ql columns fit.
bool verify_seq(int32_t ql, int32_t G, int32_t verify_rows) {
  return ql >= 2 && ql <= verify_rows && G * ql <= pa::kMaxGroup;
}

double ratio(const std::vector<int64_t>& v) {
  int64_t mx = *std::max_element(v.begin(), v.end());
  int64_t mn = *std::min_element(v.begin(), v.end());
  return mx == 0 ? 1.0 : static_cast<double>(mn) / static_cast<double>(mx);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Unmasked (row, key) pairs of a causal tile split: the rows see key counts e = e0 .. e1
// (row at position p sees keys 0 .. p, i.e. e = p + 1 keys), and within the split [kv0, kv1)
// a row with count e contributes clamp(e, kv0, kv1) - kv0 pairs. Summed in closed form:
// counts in (kv0, kv1) add e - kv0 each (an arithmetic series); counts >= kv1 add kv1 - kv0.
int64_t tile_pairs(int64_t e0, int64_t e1, int64_t kv0, int64_t kv1) {
  int64_t total = 0;
  const int64_t lo = std::max(e0, kv0 + 1), hi = std::min(e1, kv1 - 1);
  if (lo <= hi) total += (lo + hi) * (hi - lo + 1) / 2 - kv0 * (hi - lo + 1);
  const int64_t full_lo = std::max(e0, kv1);
  if (e1 >= full_lo) total += (e1 - full_lo + 1) * (kv1 - kv0);
  return total;
}

// Shared-prefix group of decode sequences first .. first+n-1 with shared length L (keys):
// per kv head and column set, the set's combine records, its shared pieces over [0, L), then
// each member's own pieces over [L, ctx). Member i of a set owns W = (S + max U) * G partial
// rows from base + i*W; piece k of a member sits at + k*G.
template <class EmitF, class CombF>
void emit_group(int32_t first, int32_t n, int32_t L, const int32_t* ctx, int32_t Hkv, int32_t G,
                int32_t dec_split, int64_t weight, EmitF& emit, CombF& combine, int64_t& parts) {
  const int32_t columns = pa::kMaxGroup / G;
  const int32_t nsets = static_cast<int32_t>(ceil_div(n, columns));
  const int64_t S = ceil_div(L, dec_split);
  for (int32_t g = 0; g < Hkv; ++g) {
    int32_t m0 = first;
    for (int32_t set = 0; set < nsets; ++set) {
      const int32_t size = n / nsets + (set < n % nsets ? 1 : 0);
      int64_t umax = 0;
      for (int32_t i = 0; i < size; ++i) umax = std::max(umax, ceil_div(ctx[m0 + i] - L, dec_split));
      const int64_t W = (S + umax) * G;
      const int64_t base = parts;
      parts += size * W;
      for (int32_t i = 0; i < size; ++i) {
        const int32_t U = static_cast<int32_t>(ceil_div(ctx[m0 + i] - L, dec_split));
        combine(pa_combine{m0 + i, 0, 1, g * G, G, static_cast<int32_t>(base + i * W),
                           static_cast<int32_t>(S) + U, 0});
      }
      for (int64_t k = 0; k < S; ++k) {
        const int32_t kv0 = static_cast<int32_t>(k * dec_split);
        const int32_t kv1 = std::min(L, kv0 + dec_split);
        emit(int64_t(kv1 - kv0) * size * G * weight,
             pa_task{PA_TASK_SHARED, m0, g, static_cast<int32_t>(W), size, kv0, kv1,
                     static_cast<int32_t>(base + k * G)});
      }
      for (int32_t i = 0; i < size; ++i) {
        const int32_t m = m0 + i;
        const int64_t U = ceil_div(ctx[m] - L, dec_split);
        for (int64_t j = 0; j < U; ++j) {
          const int32_t kv0 = L + static_cast<int32_t>(j * dec_split);
          const int32_t kv1 = std::min(ctx[m], kv0 + dec_split);
          emit(int64_t(kv1 - kv0) * G * weight,
               pa_task{PA_TASK_DECODE, m, g, 0, 1, kv0, kv1,
                       static_cast<int32_t>(base + i * W + (S + j) * G)});
        }
      }
      m0 += size;
    }
  }
}

// Emission order of the decomposition: sequences ascending; decode and verify sequences give
// kv head, then key split; prefill sequences give query head, then query tile, then key split;
// a shared-prefix group is emitted at its first member (emit_group). `emit(load, task)` and
// `combine(record)` receive every item in that order, and the partial rows are numbered in the
// same order. `pair` (NULL without sharing) holds, for s >= 1, the keys decode sequences s-1
// and s share.
template <class EmitF, class CombF>
void decompose(const pa_params* p, const int32_t* cu, const int32_t* ctx, int32_t num_seqs,
               const int32_t* pair, EmitF&& emit, CombF&& combine, int64_t* num_partials) {
  // parameters in locals: the stores of emitted records could otherwise alias them
  const int32_t Hq = p->num_q_heads, Hkv = p->num_kv_heads, G = Hq / Hkv;
  const int32_t dec_split = p->dec_split, q_tile = p->pf_q_tile, kv_split = p->pf_kv_split;
  const int64_t weight = p->decode_weight;
  const int32_t verify_rows = p->verify_rows;
  const int32_t shared_min = p->shared_min;
  const bool sharing = pair && shared_min > 0 && pa::kMaxGroup / G >= 2;
  int64_t parts = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (sharing) {
      int32_t end = s, L = INT32_MAX;
      while (end + 1 < num_seqs && pair[end + 1] >= shared_min) L = std::min(L, pair[++end]);
      if (end > s) {
        emit_group(s, end - s + 1, L, ctx, Hkv, G, dec_split, weight, emit, combine, parts);
        s = end;
        continue;
      }
    }
    const int32_t ql = cu[s + 1] - cu[s];
    const int32_t keys = ctx[s];
    const int64_t prefix = static_cast<int64_t>(keys) - ql;
    if (ql == 1 || verify_seq(ql, G, verify_rows)) {
      // decode / verify: key splits of dec_split per kv head, all ql rows and G query heads
      // in one task; its load counts the unmasked pairs of every row, times G
      const int32_t kind = ql == 1 ? PA_TASK_DECODE : PA_TASK_VERIFY;
      const int32_t nsplit = static_cast<int32_t>(ceil_div(keys, dec_split));
      const int64_t cols = static_cast<int64_t>(ql) * G;
      for (int32_t g = 0; g < Hkv; ++g) {
        int64_t first = -1;
        if (nsplit > 1) {
          first = parts;
          parts += nsplit * cols;
          combine(pa_combine{s, 0, ql, g * G, G, static_cast<int32_t>(first), nsplit, 0});
        }
        for (int32_t k = 0; k < nsplit; ++k) {
          const int32_t kv0 = k * dec_split;
          const int32_t kv1 = std::min(keys, kv0 + dec_split);
          const int32_t part = nsplit > 1 ? static_cast<int32_t>(first + k * cols) : -1;
          emit(tile_pairs(prefix + 1, prefix + ql, kv0, kv1) * G * weight,
               pa_task{kind, s, g, 0, ql, kv0, kv1, part});
        }
      }
    } else {
      // prefill: causal query tiles per query head, each split along its visible keys
      for (int32_t h = 0; h < Hq; ++h) {
        for (int32_t r0 = 0; r0 < ql; r0 += q_tile) {
          const int32_t rows = std::min(q_tile, ql - r0);
          const int64_t lim = prefix + r0 + rows;  // keys visible to the tile's last row
          const int64_t split = kv_split > 0 ? kv_split : lim;
          const int32_t nsplit = static_cast<int32_t>(ceil_div(lim, split));
          int64_t first = -1;
          if (nsplit > 1) {
            first = parts;
            parts += static_cast<int64_t>(nsplit) * rows;
            combine(pa_combine{s, r0, rows, h, 1, static_cast<int32_t>(first), nsplit, 0});
          }
          for (int32_t k = 0; k < nsplit; ++k) {
            const int64_t kv0 = k * split;
            const int64_t kv1 = std::min(lim, kv0 + split);
            const int64_t load = tile_pairs(prefix + r0 + 1, prefix + r0 + rows, kv0, kv1);
            const int32_t part =
                nsplit > 1 ? static_cast<int32_t>(first + int64_t(k) * rows) : -1;
            emit(load, pa_task{PA_TASK_PREFILL, s, h, r0, rows, static_cast<int32_t>(kv0),
                               static_cast<int32_t>(kv1), part});
          }
        }
      }
    }
  }
  *num_partials = parts;
}

// Task, combine and partial-row counts: the decomposition with counting callbacks.
void count(const pa_params* p, const int32_t* cu, const int32_t* ctx, int32_t num_seqs,
           const int32_t* pair, int64_t* nt, int64_t* nc, int64_t* np) {
  int64_t t = 0, c = 0;
  decompose(
      p, cu, ctx, num_seqs, pair, [&](int64_t, const pa_task&) { ++t; },
      [&](const pa_combine&) { ++c; }, np);
  *nt = t;
  *nc = c;
}

// Stable order of n loads, descending: an LSD radix sort on keys that hold (max_load - load)
// above the emission index, so equal loads keep emission order and the sort moves plain 64-bit
// words. The digits cover only the bits of max_load - min_load, at most 11 per pass. Returns the
// buffer (`a` or `b`, n entries each) that holds the sorted keys; the low 32 bits of each key are
// the emission index.
//
// Emission produces long runs of equal loads, so one bucket counter would take every increment
// back to back; the input is cut into kWays interleaved ranges with counters of their own (equal
// digits from an earlier range still land first, which keeps the sort stable).
uint64_t* sort_by_load_desc(const int64_t* load, uint32_t n, int64_t mn, int64_t mx, uint64_t* a,
                            uint64_t* b) {
  for (uint32_t i = 0; i < n; ++i) a[i] = (static_cast<uint64_t>(mx - load[i]) << 32) | i;
  const uint64_t span = static_cast<uint64_t>(mx - mn);
  int bits = 0;
  while (bits < 32 && (span >> bits) != 0) ++bits;
  if (bits == 0) return a;
  constexpr int kMaxBits = 11, kWays = 4;
  const int passes = (bits + kMaxBits - 1) / kMaxBits;
  const int width = (bits + passes - 1) / passes;
  const uint64_t mask = (uint64_t(1) << width) - 1;
  const uint32_t buckets = 1u << width;
  static thread_local std::vector<uint32_t> hist_store;
  hist_store.resize(size_t(kWays) << kMaxBits);
  uint32_t* hist = hist_store.data();  // [bucket][way]
  const uint32_t q = n / kWays;
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = 32 + pass * width;
    std::fill(hist, hist + size_t(kWays) * buckets, 0u);
    for (uint32_t i = 0; i < q; ++i)
      for (int w = 0; w < kWays; ++w) ++hist[((a[w * q + i] >> shift) & mask) * kWays + w];
    for (uint32_t i = kWays * q; i < n; ++i) ++hist[((a[i] >> shift) & mask) * kWays + kWays - 1];
    uint32_t run = 0;
    for (uint32_t j = 0; j < kWays * buckets; ++j) {
      const uint32_t c = hist[j];
      hist[j] = run;
      run += c;
    }
    for (uint32_t i = 0; i < q; ++i)
      for (int w = 0; w < kWays; ++w) {
        const uint64_t k = a[w * q + i];
        b[hist[((k >> shift) & mask) * kWays + w]++] = k;
      }
    for (uint32_t i = kWays * q; i < n; ++i) {
      const uint64_t k = a[i];
      b[hist[((k >> shift) & mask) * kWays + kWays - 1]++] = k;
    }
    std::swap(a, b);
  }
  return a;
}

// Scratch of the calling thread, grown on demand and reused across calls.
struct Scratch {
  std::vector<int64_t> load;
  std::vector<pa_task> task;
  std::vector<uint64_t> key, tmp;
};
Scratch& scratch() {
  static thread_local Scratch s;
  return s;
}

}  // namespace

namespace {

int check_table_inputs(const pa_params* p, const int32_t* cu, const int32_t* ctx,
                       int32_t num_seqs, const int32_t* num_tasks, const int32_t* num_combines,
                       const int32_t* num_partials) {
  if (!p || !cu || (num_seqs > 0 && !ctx) || !num_tasks || !num_combines || !num_partials)
    return set_error(PA_ERR_NULL, "build_task_table: NULL pointer");
  if (int rc = check_params(p)) return rc;
  if (num_seqs < 0) return set_error(PA_ERR_INPUT, "num_seqs %d < 0", num_seqs);
  if (cu[0] != 0) return set_error(PA_ERR_INPUT, "cu_seqlens[0] = %d, must be 0", cu[0]);
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (cu[s + 1] <= cu[s])
      return set_error(PA_ERR_INPUT, "cu_seqlens must increase strictly (seq %d)", s);
    if (ctx[s] < cu[s + 1] - cu[s])
      return set_error(PA_ERR_INPUT, "context_lens[%d] = %d is shorter than its %d query rows",
                       s, ctx[s], cu[s + 1] - cu[s]);
  }
  return PA_OK;
}

int build_table(const pa_params* p, const int32_t* cu, const int32_t* ctx, int32_t num_seqs,
                const int32_t* pair, pa_task* tasks, int32_t tasks_cap, int32_t* num_tasks,
                pa_combine* combines, int32_t combines_cap, int32_t* num_combines,
                int32_t* num_partials, double* balance, uint32_t* task_kinds);

}  // namespace

// Dynamic Decomposer + load-sorted reorder (XY-Serve page, sections 2.2 and 4.4).
extern "C" int build_task_table(const pa_params* p, const int32_t* cu, const int32_t* ctx,
                                int32_t num_seqs, pa_task* tasks, int32_t tasks_cap,
                                int32_t* num_tasks, pa_combine* combines, int32_t combines_cap,
                                int32_t* num_combines, int32_t* num_partials, double* balance,
                                uint32_t* task_kinds) {
  if (int rc = check_table_inputs(p, cu, ctx, num_seqs, num_tasks, num_combines, num_partials))
    return rc;
  if (p->shared_min > 0)
    return set_error(PA_ERR_INPUT,
                     "shared_min > 0 needs the block table: call build_task_table_shared");
  return build_table(p, cu, ctx, num_seqs, nullptr, tasks, tasks_cap, num_tasks, combines,
                     combines_cap, num_combines, num_partials, balance, task_kinds);
}

// The same plus shared-prefix groups (XY-Serve page, automatic prefix cache; ATB page, KV cache
// reuse), found from a host copy of the block table.
extern "C" int build_task_table_shared(const pa_params* p, const int32_t* cu, const int32_t* ctx,
                                       int32_t num_seqs, const int32_t* bt, int32_t width,
                                       pa_task* tasks, int32_t tasks_cap, int32_t* num_tasks,
                                       pa_combine* combines, int32_t combines_cap,
                                       int32_t* num_combines, int32_t* num_partials,
                                       double* balance, uint32_t* task_kinds) {
  if (int rc = check_table_inputs(p, cu, ctx, num_seqs, num_tasks, num_combines, num_partials))
    return rc;
  if (p->shared_min == 0)
    return build_table(p, cu, ctx, num_seqs, nullptr, tasks, tasks_cap, num_tasks, combines,
                       combines_cap, num_combines, num_partials, balance, task_kinds);
  if (num_seqs > 0 && !bt)
    return set_error(PA_ERR_NULL, "build_task_table_shared: block_table is NULL");
  const int32_t bs = p->block_size;
  for (int32_t s = 0; s < num_seqs; ++s)
    if ((ctx[s] + bs - 1) / bs > width)
      return set_error(PA_ERR_SHAPE, "seq %d needs %d blocks, table has %d columns", s,
                       (ctx[s] + bs - 1) / bs, width);
  // keys that decode neighbours s-1 and s read from the same physical blocks
  static thread_local std::vector<int32_t> pair;
  pair.assign(static_cast<size_t>(std::max(num_seqs, 1)), 0);
  for (int32_t s = 1; s < num_seqs; ++s) {
    if (cu[s + 1] - cu[s] != 1 || cu[s] - cu[s - 1] != 1) continue;
    const int32_t need = std::min((ctx[s - 1] + bs - 1) / bs, (ctx[s] + bs - 1) / bs);
    const int32_t* a = bt + static_cast<int64_t>(s - 1) * width;
    const int32_t* b = bt + static_cast<int64_t>(s) * width;
    int32_t common = 0;
    while (common < need && a[common] == b[common]) ++common;
    // logical block (ctx-1)/bs receives the sequence's new row in this step
    if (common > std::min((ctx[s - 1] - 1) / bs, (ctx[s] - 1) / bs))
      return set_error(PA_ERR_INPUT,
                       "sequences %d and %d share block_table[.][%d] = %d, which receives a "
                       "new row", s - 1, s, std::min((ctx[s - 1] - 1) / bs, (ctx[s] - 1) / bs),
                       a[std::min((ctx[s - 1] - 1) / bs, (ctx[s] - 1) / bs)]);
    pair[s] = static_cast<int32_t>(int64_t(common) * bs / pa::kSplitQuantum * pa::kSplitQuantum);
  }
  return build_table(p, cu, ctx, num_seqs, pair.data(), tasks, tasks_cap, num_tasks, combines,
                     combines_cap, num_combines, num_partials, balance, task_kinds);
}

namespace {

int build_table(const pa_params* p, const int32_t* cu, const int32_t* ctx, int32_t num_seqs,
                const int32_t* pair, pa_task* tasks, int32_t tasks_cap, int32_t* num_tasks,
                pa_combine* combines, int32_t combines_cap, int32_t* num_combines,
                int32_t* num_partials, double* balance, uint32_t* task_kinds) {
  int64_t nt = 0, nc = 0, np = 0;
  count(p, cu, ctx, num_seqs, pair, &nt, &nc, &np);
  if (nt > INT32_MAX || nc > INT32_MAX || np > INT32_MAX)
    return set_error(PA_ERR_SHAPE, "task table exceeds int32 indexing");
  *num_tasks = static_cast<int32_t>(nt);
  *num_combines = static_cast<int32_t>(nc);
  *num_partials = static_cast<int32_t>(np);
  if (task_kinds) *task_kinds = 0;
  if (nt > tasks_cap || nc > combines_cap) {
    if (balance) balance[0] = balance[1] = 0.0;
    return set_error(PA_ERR_CAPACITY, "need %lld tasks (cap %d) and %lld combines (cap %d)",
                     static_cast<long long>(nt), tasks_cap, static_cast<long long>(nc),
                     combines_cap);
  }
  if (nt > 0 && !tasks) return set_error(PA_ERR_NULL, "build_task_table: tasks is NULL");
  if (nc > 0 && !combines) return set_error(PA_ERR_NULL, "build_task_table: combines is NULL");

  Scratch& sc = scratch();
  if (sc.load.size() < static_cast<size_t>(nt)) {
    sc.load.resize(nt);
    sc.task.resize(nt);
    sc.key.resize(nt);
    sc.tmp.resize(nt);
  }
  int64_t* loads = sc.load.data();
  pa_task* emitted = sc.task.data();
  int64_t nti = 0, nci = 0, parts = 0;
  int64_t mn = INT64_MAX, mx = 0;
  uint32_t kinds = 0;
  decompose(
      p, cu, ctx, num_seqs, pair,
      [&](int64_t load, const pa_task& t) {
        if (nti < nt) {
          loads[nti] = load;
          emitted[nti] = t;
          mn = std::min(mn, load);
          mx = std::max(mx, load);
          kinds |= 1u << t.kind;
        }
        ++nti;
      },
      [&](const pa_combine& c) {
        if (nci < nc) combines[nci] = c;
        ++nci;
      },
      &parts);
  if (nti != nt || nci != nc || parts != np)
    return set_error(PA_ERR_SHAPE, "build_task_table: internal count mismatch");
  const uint64_t* order;
  if (nt == 0 || static_cast<uint64_t>(mx - mn) < (uint64_t(1) << 32)) {
    order = sort_by_load_desc(loads, static_cast<uint32_t>(nt), mn, mx, sc.key.data(),
                              sc.tmp.data());
  } else {
    // loads spread over more than 2^32 (a 128-row tile over tens of millions of keys): a stable
    // comparison sort of the emission indices instead of the packed keys
    uint64_t* idx = sc.key.data();
    for (int64_t i = 0; i < nt; ++i) idx[i] = static_cast<uint64_t>(i);
    std::stable_sort(idx, idx + nt,
                     [loads](uint64_t x, uint64_t y) { return loads[x] > loads[y]; });
    order = idx;
  }
  for (int64_t i = 0; i < nt; ++i) tasks[i] = emitted[static_cast<uint32_t>(order[i])];
  if (task_kinds) *task_kinds = kinds;
  if (balance) {
    const int32_t W = p->num_workers;
    std::vector<int64_t> snake(W, 0), modulo(W, 0);
    for (int64_t i = 0; i < nt; ++i) {
      const int64_t ld = loads[static_cast<uint32_t>(order[i])];
      const size_t rnd = i / W, pos = i % W;
      snake[rnd % 2 == 0 ? pos : W - 1 - pos] += ld;
      modulo[i % W] += ld;
    }
    balance[0] = ratio(snake);
    balance[1] = ratio(modulo);
  }
  return pa::clear_error();
}

}  // namespace

extern "C" size_t pa_workspace_bytes(int32_t num_partials, int32_t head_dim) {
  if (num_partials <= 0 || head_dim <= 0) return 0;
  // [num_partials, D] fp32 accumulators, then [num_partials, 2] fp32 (running max, sum);
  // the second region starts on a 256-byte boundary
  size_t acc = static_cast<size_t>(num_partials) * head_dim * sizeof(float);
  acc = (acc + 255) & ~size_t(255);
  size_t ml = static_cast<size_t>(num_partials) * 2 * sizeof(float);
  return (acc + ml + 255) & ~size_t(255);
}

// Debug check of a host block table (cann-recipes-infer page, section 4.4, first check).
extern "C" int pa_validate_block_table(const int32_t* bt, int32_t width, const int32_t* ctx,
                                       int32_t num_seqs, int32_t num_blocks, int32_t bs) {
  if ((num_seqs > 0 && (!bt || !ctx)))
    return set_error(PA_ERR_NULL, "pa_validate_block_table: NULL pointer");
  if (!pa::block_size_ok(bs))
    return set_error(PA_ERR_BLOCK_SIZE, "block_size %d is not a power of two in [16, 256]", bs);
  if (num_blocks < 0 || width < 0 || num_seqs < 0)
    return set_error(PA_ERR_SHAPE, "negative size");
  std::vector<int32_t> owner(static_cast<size_t>(num_blocks), -1);
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (ctx[s] < 0) return set_error(PA_ERR_INPUT, "context_lens[%d] = %d < 0", s, ctx[s]);
    const int32_t need = (ctx[s] + bs - 1) / bs;
    if (need > width)
      return set_error(PA_ERR_SHAPE, "seq %d needs %d blocks, table has %d columns", s, need,
                       width);
    for (int32_t j = 0; j < need; ++j) {
      const int32_t b = bt[static_cast<int64_t>(s) * width + j];
      if (b < 0 || b >= num_blocks)
        return set_error(PA_ERR_INPUT, "block_table[%d][%d] = %d outside [0, %d)", s, j, b,
                         num_blocks);
      if (owner[b] >= 0)
        return set_error(PA_ERR_INPUT, "physical block %d claimed by seq %d and seq %d", b,
                         owner[b], s);
      owner[b] = s;
    }
  }
  return pa::clear_error();
}

// Linear decomposition for SmoothGEMM (XY-Serve page, section 4.4, decompose_linear; section
// 2.2, SmoothGEMM): output blocks of tile x tile, K pieces of k_split, loads of
// rows * cols * k, stable sort by load, descending.
extern "C" int build_gemm_table(const pa_gemm_params* p, int32_t M, int32_t N, int32_t K,
                                pa_gemm_task* tasks, int32_t tasks_cap, int32_t* num_tasks,
                                pa_gemm_reduce* reduces, int32_t reduces_cap,
                                int32_t* num_reduces, int32_t* num_slots, double* balance) {
  if (!p || !num_tasks || !num_reduces || !num_slots)
    return set_error(PA_ERR_NULL, "build_gemm_table: NULL pointer");
  if (p->tile != 128 && p->tile != 256)
    return set_error(PA_ERR_SHAPE, "tile %d must be 128 or 256", p->tile);
  if (p->k_split < 0 || p->k_split % pa::kSplitQuantum)
    return set_error(PA_ERR_SHAPE, "k_split %d must be 0 or a positive multiple of %d",
                     p->k_split, pa::kSplitQuantum);
  if (p->num_workers < 1) return set_error(PA_ERR_SHAPE, "num_workers must be >= 1");
  if (p->tail_split != 0 && (p->tail_split != 1 || p->k_split != 0))
    return set_error(PA_ERR_SHAPE, "tail_split must be 0, or 1 with k_split 0");
  if (M < 0 || N < 0 || K < 0) return set_error(PA_ERR_SHAPE, "negative size");
  if (K == 0 && M > 0 && N > 0)
    return set_error(PA_ERR_SHAPE, "K must be >= 1 for a non-empty product");
  const int64_t tile = p->tile;
  const int64_t mb = (M + tile - 1) / tile, nb = (N + tile - 1) / tile;
  // output blocks in emission order (m block, n block); none when any size is zero
  const int64_t T = (K > 0 && M > 0 && N > 0) ? mb * nb : 0;
  if (T > INT32_MAX) return set_error(PA_ERR_SHAPE, "too many tasks");
  auto rows_of = [&](int64_t b) { return std::min<int64_t>(tile, M - (b / nb) * tile); };
  auto cols_of = [&](int64_t b) { return std::min<int64_t>(tile, N - (b % nb) * tile); };
  // K piece length of each block: k_split, or all of K; with tail_split the blocks of the last,
  // partial round of W workers (the last r = T mod W of the whole blocks in load order) are cut
  // into p = min(W / r, ceil(K / 64)) pieces when p >= 2
  const int64_t whole_split = p->k_split > 0 ? p->k_split : std::max<int64_t>(K, 1);
  std::vector<int64_t> split(static_cast<size_t>(T), whole_split);
  if (p->tail_split && T > 0) {
    const int64_t W = p->num_workers, r = T % W;
    const int64_t pieces = r ? std::min<int64_t>(W / r, (K + pa::kSplitQuantum - 1) / pa::kSplitQuantum) : 1;
    if (pieces >= 2) {
      const int64_t kp = ((K + pieces - 1) / pieces + pa::kSplitQuantum - 1) / pa::kSplitQuantum *
                         pa::kSplitQuantum;
      std::vector<uint32_t> whole(static_cast<size_t>(T));
      std::iota(whole.begin(), whole.end(), 0u);
      std::stable_sort(whole.begin(), whole.end(), [&](uint32_t x, uint32_t y) {
        return rows_of(x) * cols_of(x) > rows_of(y) * cols_of(y);
      });
      for (int64_t i = T - r; i < T; ++i) split[whole[static_cast<size_t>(i)]] = kp;
    }
  }
  int64_t nt = 0, nr = 0, ns = 0;
  for (int64_t b = 0; b < T; ++b) {
    const int64_t nk = (K + split[static_cast<size_t>(b)] - 1) / split[static_cast<size_t>(b)];
    nt += nk;
    if (nk > 1) {
      ++nr;
      ns += nk;
    }
  }
  if (nt > INT32_MAX) return set_error(PA_ERR_SHAPE, "too many tasks");
  *num_tasks = static_cast<int32_t>(nt);
  *num_reduces = static_cast<int32_t>(nr);
  *num_slots = static_cast<int32_t>(ns);
  if (nt > tasks_cap || nr > reduces_cap)
    return set_error(PA_ERR_CAPACITY, "build_gemm_table: need %lld tasks and %lld reduces",
                     static_cast<long long>(nt), static_cast<long long>(nr));
  if ((nt > 0 && !tasks) || (nr > 0 && !reduces))
    return set_error(PA_ERR_NULL, "build_gemm_table: NULL output buffer");
  std::vector<pa_gemm_task> emitted;
  std::vector<int64_t> load;
  emitted.reserve(static_cast<size_t>(nt));
  load.reserve(static_cast<size_t>(nt));
  int32_t slot = 0, r = 0;
  for (int64_t b = 0; b < T; ++b) {
    const int64_t m0 = (b / nb) * tile, n0 = (b % nb) * tile;
    const int32_t rows = static_cast<int32_t>(rows_of(b)), cols = static_cast<int32_t>(cols_of(b));
    const int64_t sp = split[static_cast<size_t>(b)];
    const int64_t nk = (K + sp - 1) / sp;
    const int32_t first = nk > 1 ? slot : -1;
    if (nk > 1) {
      reduces[r++] = pa_gemm_reduce{static_cast<int32_t>(m0), rows, static_cast<int32_t>(n0),
                                    cols, first, static_cast<int32_t>(nk), 0, 0};
      slot += static_cast<int32_t>(nk);
    }
    for (int64_t j = 0; j < nk; ++j) {
      const int64_t k0 = j * sp, k1 = std::min<int64_t>(K, k0 + sp);
      emitted.push_back(pa_gemm_task{static_cast<int32_t>(m0), rows, static_cast<int32_t>(n0),
                                     cols, static_cast<int32_t>(k0), static_cast<int32_t>(k1),
                                     nk > 1 ? first + static_cast<int32_t>(j) : -1, 0});
      load.push_back(int64_t(rows) * cols * (k1 - k0));
    }
  }
  std::vector<uint32_t> order(emitted.size());
  std::iota(order.begin(), order.end(), 0u);
  std::stable_sort(order.begin(), order.end(),
                   [&](uint32_t x, uint32_t y) { return load[x] > load[y]; });
  for (size_t i = 0; i < order.size(); ++i) tasks[i] = emitted[order[i]];
  if (balance) {
    const int64_t W = p->num_workers;
    std::vector<int64_t> snake(static_cast<size_t>(W), 0), modulo(static_cast<size_t>(W), 0);
    for (size_t i = 0; i < order.size(); ++i) {
      const int64_t rnd = static_cast<int64_t>(i) / W, pos = static_cast<int64_t>(i) % W;
      snake[static_cast<size_t>(rnd % 2 == 0 ? pos : W - 1 - pos)] += load[order[i]];
      modulo[static_cast<size_t>(pos)] += load[order[i]];
    }
    balance[0] = ratio(snake);
    balance[1] = ratio(modulo);
  }
  return pa::clear_error();
}
