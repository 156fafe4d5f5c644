// Randomised calls of the host entry points (plan builders, balance, draft
// tree, block pool) with valid and invalid descriptions, built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.
// Every call must either succeed or return a status; the sanitizers report any
// out-of-bounds access, leak or undefined operation on the way.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>
#include "tree_attn.h"
static std::mt19937 rng(12345);
static int U(int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); }
int main(int argc, char** argv) {
  int iters = argc > 1 ? atoi(argv[1]) : 2000;
  int ok = 0, err = 0;
  for (int it = 0; it < iters; ++it) {
    // prefill
    {
      int np = U(0, 3);
      std::vector<int32_t> P(np), N(np), L, C;
      for (int p = 0; p < np; ++p) {
        P[p] = U(-1, 300); N[p] = U(0, 5);
        for (int k = 0; k < N[p]; ++k) { L.push_back(U(-1, 40)); C.push_back(U(0, 200)); }
      }
      ta_plan* pl = nullptr;
      int rc = tree_attn_plan_prefill(P.data(), N.data(), L.data(), C.data(), np, &pl);
      if (rc == TA_OK) { ++ok; if (U(0, 1)) tree_attn_plan_balance(pl, U(1, 8), U(1, 600)); tree_attn_plan_destroy(pl); } else ++err;
    }
    // decode (single, multi, paged)
    {
      int np = U(1, 3);
      std::vector<int32_t> P(np), N(np), L;
      for (int p = 0; p < np; ++p) { P[p] = U(0, 3000); N[p] = U(0, 4); for (int k = 0; k < N[p]; ++k) L.push_back(U(0, 80)); }
      int nb = U(0, 6);
      std::vector<int32_t> bp(nb), br(nb), s(nb), kq(nb);
      int page = 0;
      for (int b = 0; b < nb; ++b) { page = std::min(np - 1, page + U(0, 1)); bp[b] = page; br[b] = U(-1, N[page] + 1); s[b] = U(-1, 3000); kq[b] = U(0, 150); }
      ta_plan* pl = nullptr;
      int mode = U(0, 2);
      int rc;
      if (mode == 0) rc = tree_attn_plan_decode(P.data(), N.data(), L.data(), np, bp.data(), br.data(), s.data(), nb, &pl);
      else if (mode == 1) rc = tree_attn_plan_decode_multi(P.data(), N.data(), L.data(), np, bp.data(), br.data(), s.data(), kq.data(), nb, &pl);
      else {
        int bs = 64 * U(0, 3);
        int ncb = U(0, 400);
        std::vector<int32_t> mb, sb; std::vector<int64_t> mo(np + 1, 0), so(nb + 1, 0);
        for (int p = 0; p < np; ++p) { int n = U(0, 100); for (int j = 0; j < n; ++j) mb.push_back(U(-1, ncb)); mo[p + 1] = mo[p] + n; }
        for (int b = 0; b < nb; ++b) { int n = U(0, 100); for (int j = 0; j < n; ++j) sb.push_back(U(-1, ncb)); so[b + 1] = so[b] + n; }
        rc = tree_attn_plan_decode_paged(P.data(), N.data(), L.data(), np, bp.data(), br.data(), s.data(), U(0,1) ? kq.data() : nullptr, nb, bs, ncb,
                                         mb.data(), mo.data(), sb.data(), so.data(), &pl);
      }
      if (rc == TA_OK) { ++ok; tree_attn_plan_destroy(pl); } else ++err;
    }
    // verify (plain and paged) + accept scratch
    {
      int np = U(1, 3), nb = U(0, 5);
      std::vector<int32_t> ctx(np), bp(nb), nn(nb), par;
      for (int p = 0; p < np; ++p) ctx[p] = U(-1, 3000);
      int page = 0;
      for (int b = 0; b < nb; ++b) {
        page = std::min(np - 1, page + U(0, 1)); bp[b] = page; nn[b] = U(0, 66);
        for (int i = 0; i < nn[b]; ++i) par.push_back(U(-2, i));
      }
      ta_plan* pl = nullptr;
      int rc;
      if (U(0, 1)) rc = tree_attn_plan_verify(ctx.data(), np, bp.data(), nn.data(), par.data(), nb, &pl);
      else {
        int bs = 64 * U(1, 2), ncb = U(0, 200);
        std::vector<int32_t> cb; std::vector<int64_t> co(np + 1, 0);
        for (int p = 0; p < np; ++p) { int n = U(0, 60); for (int j = 0; j < n; ++j) cb.push_back(U(-1, ncb)); co[p + 1] = co[p] + n; }
        rc = tree_attn_plan_verify_paged(ctx.data(), np, bp.data(), nn.data(), par.data(), nb, bs, ncb, cb.data(), co.data(), &pl);
      }
      if (rc == TA_OK) { ++ok; if (U(0, 1)) tree_attn_plan_balance(pl, U(1, 8), U(1, 600)); tree_attn_plan_destroy(pl); } else ++err;
    }
    // draft tree
    {
      int na = U(0, 10), nd = U(0, 4), w = U(0, 4), mn = U(0, 70), md = U(0, 9);
      std::vector<int32_t> acc(na), dl(nd), dr;
      for (auto& a : acc) a = U(0, 3);
      for (int d = 0; d < nd; ++d) { dl[d] = U(0, 60); for (int j = 0; j < dl[d]; ++j) dr.push_back(U(0, 3)); }
      std::vector<int32_t> tok(std::max(mn, 0)), par(std::max(mn, 0));
      int32_t n = 0;
      int rc = tree_attn_draft_tree(acc.data(), na, dr.data(), dl.data(), nd, w, mn, md, tok.data(), par.data(), &n);
      if (rc == TA_OK) { ++ok; if (n > mn) { printf("draft overflow\n"); return 1; } } else ++err;
    }
    // pool
    {
      ta_kv_pool* pool = nullptr;
      if (tree_attn_pool_create(U(0, 30), U(1, 70), &pool) == TA_OK) {
        std::vector<int32_t> seqs;
        for (int k = 0; k < 60; ++k) {
          int op = U(0, 4);
          int32_t s = seqs.empty() ? -1 : seqs[U(0, (int)seqs.size() - 1)];
          if (op == 0) { int32_t id; if (tree_attn_pool_new_seq(pool, &id) == TA_OK) seqs.push_back(id); }
          else if (op == 1) { int n = U(-1, 200); std::vector<int64_t> sl(std::max(n, 0)); tree_attn_pool_append(pool, s, n, sl.data()); }
          else if (op == 2) { int32_t c; if (tree_attn_pool_fork(pool, s, U(-1, 200), &c) == TA_OK) seqs.push_back(c); }
          else if (op == 3) { tree_attn_pool_release(pool, s); }
          else { std::vector<int32_t> v(8), o(8); int32_t vt, ot; tree_attn_pool_table(pool, s, v.data(), 8, &vt, o.data(), 8, &ot); }
        }
        int32_t fr; std::vector<int32_t> refs(64); tree_attn_pool_refs(pool, refs.data(), 64, &fr);
        tree_attn_pool_destroy(pool);
        ++ok;
      }
    }
  }
  printf("ok=%d err=%d\n", ok, err);
  return 0;
}
