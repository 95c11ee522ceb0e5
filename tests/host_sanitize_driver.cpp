// Host-only driver for the table builders under AddressSanitizer and UndefinedBehaviorSanitizer:
// random batches (decode, draft and prefill rows, shared leading blocks), every tiling knob,
// undersized then exact output buffers (heap-allocated, so an overrun is reported), and random
// Linear shapes for the GEMM table. Prints "ok <n>, rejected inputs <m>"; exits non-zero on a
// failed exact-size call or a missing capacity error. Iteration counts: argv[1], argv[2].
#include <cstdio>
#include <algorithm>
#include <cstdlib>
#include <random>
#include <vector>
#include "pagedattn.h"

static std::mt19937 rng(1234);
static int ri(int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); }

int main(int argc, char** argv) {
  const int n_attn = argc > 1 ? std::atoi(argv[1]) : 3000;
  const int n_gemm = argc > 2 ? std::atoi(argv[2]) : 2000;
  int ok = 0, errs = 0;
  for (int it = 0; it < n_attn; ++it) {
    pa_params p{};
    int hkv = 1 << ri(0, 3), g = 1 << ri(0, 4);
    p.num_q_heads = hkv * g; p.num_kv_heads = hkv; p.head_dim = ri(0, 1) ? 64 : 128;
    p.block_size = 16 << ri(0, 4);
    p.dec_split = 64 * ri(1, 20); p.pf_q_tile = ri(1, 128); p.pf_kv_split = ri(0, 1) ? 0 : 64 * ri(1, 10);
    p.num_workers = ri(1, 600); p.decode_weight = ri(1, 40);
    p.verify_rows = ri(0, 1) ? 0 : ri(2, 16); p.shared_min = ri(0, 1) ? 0 : 64 * ri(1, 4);
    int n = ri(0, 40);
    std::vector<int32_t> ql(n), ctx(n), cu(n + 1);
    for (int i = 0; i < n; ++i) {
      int kind = ri(0, 2);
      ql[i] = kind == 0 ? 1 : (kind == 1 ? ri(2, 5) : ri(5, 600));
      ctx[i] = ql[i] + ri(0, 5000);
    }
    if (pa_pack_seqlens(n ? ql.data() : nullptr, n, cu.data()) != PA_OK) { ++errs; continue; }
    // block table: runs of neighbours sharing leading blocks
    int bs = p.block_size, maxb = 1;
    for (int i = 0; i < n; ++i) maxb = std::max(maxb, (ctx[i] + bs - 1) / bs);
    std::vector<int32_t> bt(static_cast<size_t>(n) * maxb, -1);
    int next = 0;
    for (int i = 0; i < n; ++i) {
      int need = (ctx[i] + bs - 1) / bs;
      int share = (i > 0 && ql[i] == 1 && ql[i - 1] == 1 && ri(0, 1)) ? ri(0, need - 1) : 0;
      int prev_need = i > 0 ? (ctx[i - 1] + bs - 1) / bs : 0;
      share = std::min(share, std::max(0, prev_need - 1));
      for (int b = 0; b < need; ++b)
        bt[static_cast<size_t>(i) * maxb + b] = b < share ? bt[static_cast<size_t>(i - 1) * maxb + b] : next++;
    }
    int32_t nt = 0, nc = 0, np = 0;
    double bal[2];
    uint32_t kinds = 0;
    int rc0 = p.shared_min
                  ? build_task_table_shared(&p, cu.data(), ctx.data(), n, bt.data(), maxb, nullptr, 0, &nt,
                                            nullptr, 0, &nc, &np, bal, &kinds)
                  : build_task_table(&p, cu.data(), ctx.data(), n, nullptr, 0, &nt, nullptr, 0, &nc, &np,
                                     bal, &kinds);
    if (rc0 != PA_OK && rc0 != PA_ERR_CAPACITY) { ++errs; continue; }
    // undersized, then exact buffers
    for (int pass = 0; pass < 2; ++pass) {
      int tc = pass == 0 ? std::max(0, nt - 1) : nt, cc = pass == 0 ? std::max(0, nc - 1) : nc;
      pa_task* t = static_cast<pa_task*>(std::malloc(sizeof(pa_task) * std::max(tc, 1)));
      pa_combine* c = static_cast<pa_combine*>(std::malloc(sizeof(pa_combine) * std::max(cc, 1)));
      int32_t nt2, nc2, np2;
      int rc = p.shared_min
                   ? build_task_table_shared(&p, cu.data(), ctx.data(), n, bt.data(), maxb, t, tc, &nt2, c, cc,
                                             &nc2, &np2, bal, &kinds)
                   : build_task_table(&p, cu.data(), ctx.data(), n, t, tc, &nt2, c, cc, &nc2, &np2, bal, &kinds);
      if (pass == 1 && rc != PA_OK) { std::printf("exact-size call failed it=%d rc=%d %s\n", it, rc, pa_last_error()); return 1; }
      if (pass == 0 && (nt > 0 || nc > 0) && (tc < nt || cc < nc) && rc != PA_ERR_CAPACITY) {
        std::printf("undersized call did not report capacity it=%d rc=%d\n", it, rc); return 1;
      }
      std::free(t); std::free(c);
    }
    std::vector<int32_t> bt_ok(bt);
    pa_validate_block_table(bt_ok.data(), maxb, ctx.data(), n, next, bs);
    ++ok;
  }
  // GEMM tables
  for (int it = 0; it < n_gemm; ++it) {
    pa_gemm_params gp{};
    gp.tile = ri(0, 1) ? 128 : 256; gp.k_split = ri(0, 1) ? 0 : 64 * ri(1, 16);
    gp.num_workers = ri(1, 600); gp.tail_split = gp.k_split == 0 ? ri(0, 1) : 0;
    int M = ri(0, 5000), N = ri(0, 3000), K = ri(1, 9000);
    int32_t nt = 0, nr = 0, ns = 0; double bal[2];
    int rc0 = build_gemm_table(&gp, M, N, K, nullptr, 0, &nt, nullptr, 0, &nr, &ns, bal);
    if (rc0 != PA_OK && rc0 != PA_ERR_CAPACITY) { ++errs; continue; }
    for (int pass = 0; pass < 2; ++pass) {
      int tc = pass == 0 ? std::max(0, nt - 1) : nt, rcap = pass == 0 ? std::max(0, nr - 1) : nr;
      pa_gemm_task* t = static_cast<pa_gemm_task*>(std::malloc(sizeof(pa_gemm_task) * std::max(tc, 1)));
      pa_gemm_reduce* r = static_cast<pa_gemm_reduce*>(std::malloc(sizeof(pa_gemm_reduce) * std::max(rcap, 1)));
      int32_t a, b, c;
      int rc = build_gemm_table(&gp, M, N, K, t, tc, &a, r, rcap, &b, &c, bal);
      if (pass == 1 && rc != PA_OK) { std::printf("gemm exact-size call failed it=%d rc=%d\n", it, rc); return 1; }
      std::free(t); std::free(r);
    }
    ++ok;
  }
  std::printf("ok %d, rejected inputs %d\n", ok, errs);
  return 0;
}
