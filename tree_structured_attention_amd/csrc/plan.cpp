// Host plan builder: turns a page/branch/tree description into per-row key
// bounds, tree bitmasks and an ordered work list.  Integer work only; no GPU.
//
// Visibility it encodes (sources named in the public header):
//   prefill  row in the main stream of a page: keys [page_base, row]
//            row Y_k[t]: keys [page_base, page_base + P + L_<=k) and
//            [start of Y_k, row]   (ancestor sets of the PaDoc summary,
//            "Training paradigm")
//   decode   branch (page p, region k, s_k): main_p[0, P + L_<=k) plus its
//            own s_k + 1 suffix tokens (PaDoc summary, "Inference")
//   verify   node i: its page's context plus anc*(i) inside its tree (HSD
//            notes, key design 3 (b))
// With the packed order [X | B_1..B_N | Y_1..Y_N] a row's visible keys are
// at most two contiguous intervals, so no mask memory is needed outside the
// 64-node draft trees.
#include <algorithm>
#include <memory>
#include <climits>
#include <cstring>
#include <numeric>

#include "ta_internal.h"

namespace ta {

namespace {

constexpr int64_t kMax32 = INT32_MAX;

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

int64_t item_cost(const WorkItem& w) {
  // a workgroup's time follows its tiles, whatever its row count
  return int64_t(w.tile_hi - w.tile_lo) * 64 + w.nrows;
}

// Longest first, so that the long tiles start early and the short ones fill
// the tail; ties keep plan order.
void order_work(std::vector<WorkItem>& w) {
  std::stable_sort(w.begin(), w.end(),
                   [](const WorkItem& x, const WorkItem& y) { return item_cost(x) > item_cost(y); });
}

// Prefill: pages in order, each page's items longest first.  Every item of
// a KV head runs on that head's XCD (workgroup x = item * Hkv + head, and
// workgroups go round-robin over the 8 XCDs), so with this order an XCD's
// slots work on one or two pages at a time and the K/V those row tiles
// re-read stays in its 4 MB L2.  Longest first over all pages mixed the
// row tiles of every page on each XCD: 4.4 GB of HBM traffic per launch
// for the 8-page batch (0.95 GB algorithmic) against 1.28 GB in page order.
void order_work_paged(std::vector<WorkItem>& w, const std::vector<int64_t>& pages5) {
  std::vector<int64_t> base;
  for (size_t i = 0; i < pages5.size(); i += 5) base.push_back(pages5[i]);
  auto page_of = [&](int32_t row) {
    return int(std::upper_bound(base.begin(), base.end(), int64_t(row)) - base.begin()) - 1;
  };
  std::stable_sort(w.begin(), w.end(), [&](const WorkItem& x, const WorkItem& y) {
    const int px = page_of(x.row0), py = page_of(y.row0);
    if (px != py) return px < py;
    return item_cost(x) > item_cost(y);
  });
}

WorkItem make_item(int64_t row0, int64_t nrows, int64_t a_lo, int64_t a_full, int64_t a_hi,
                   int64_t b_lo, int64_t b_hi, int64_t out, int32_t flags) {
  WorkItem w{};
  w.row0 = int32_t(row0);
  w.nrows = int32_t(nrows);
  w.a_lo = int32_t(a_lo);
  w.a_full = int32_t(std::max(a_lo, std::min(a_full, a_hi)));
  w.a_hi = int32_t(a_hi);
  w.b_lo = int32_t(b_lo);
  w.b_hi = int32_t(std::max(b_lo, b_hi));
  w.out = int32_t(out);
  w.flags = flags;
  w.b_full = w.b_lo;
  w.tile_lo = 0;
  w.tile_hi = int32_t(item_tiles(w));
  return w;
}

// Block tables of paged plans.  A sequence i of `len(i)` tokens reads token t
// from cache row blocks[off[i] + t / bs] * bs + t % bs.  Block sizes are
// multiples of the 64-key tile, so no tile straddles two blocks.
struct Paging {
  int32_t bs = 0, n_cache_blocks = 0;
  const int32_t* blocks = nullptr;
  const int64_t* off = nullptr;
  bool on() const { return bs > 0; }
};

int64_t round_tile(int64_t n) { return (n + kKeyTile - 1) / kKeyTile * kKeyTile; }

int check_paging(const Paging& pg, int32_t n_seq, const std::vector<int64_t>& len, const char* who) {
  if (pg.bs < kKeyTile || pg.bs % kKeyTile != 0)
    return fail(TA_ERR_INVALID_ARG, std::string(who) + ": block_size must be a positive multiple of 64");
  if (pg.n_cache_blocks < 0 || int64_t(pg.n_cache_blocks) * pg.bs >= kMax32)
    return fail(TA_ERR_CAPACITY, std::string(who) + ": cache rows must stay below 2^31");
  if (n_seq > 0 && (!pg.off || !pg.blocks)) return fail(TA_ERR_INVALID_ARG, std::string(who) + ": NULL block table");
  for (int32_t i = 0; i < n_seq; ++i) {
    const int64_t need = (len[i] + pg.bs - 1) / pg.bs;
    if (pg.off[i] < 0 || pg.off[i + 1] - pg.off[i] < need)
      return fail(TA_ERR_INVALID_ARG, std::string(who) + ": a block table is shorter than its sequence");
    for (int64_t j = 0; j < need; ++j) {
      const int32_t b = pg.blocks[pg.off[i] + j];
      if (b < 0 || b >= pg.n_cache_blocks) return fail(TA_ERR_INVALID_ARG, std::string(who) + ": block id out of range");
    }
  }
  return TA_OK;
}

// Physical row of every tile of the sequences laid out from virtual bases.
void fill_tiles(const Paging& pg, int32_t n_seq, const std::vector<int64_t>& len, const std::vector<int64_t>& vbase,
                int64_t v_total, std::vector<int32_t>& tiles) {
  tiles.assign(size_t(v_total / kKeyTile), 0);
  for (int32_t i = 0; i < n_seq; ++i)
    for (int64_t t = 0; t < len[i]; t += kKeyTile)
      tiles[size_t((vbase[i] + t) / kKeyTile)] = pg.blocks[pg.off[i] + t / pg.bs] * pg.bs + int32_t(t % pg.bs);
}

}  // namespace

int64_t item_tiles(const WorkItem& w) {
  return (int64_t(w.a_hi - w.a_lo) + kKeyTile - 1) / kKeyTile + (int64_t(w.b_hi - w.b_lo) + kKeyTile - 1) / kKeyTile;
}

void pack_blob(ta_plan* p) {
  DeviceLayout L;
  int64_t off = 0;
  L.work = off;
  off = align256(off + int64_t(p->work.size() * sizeof(WorkItem)));
  L.row_a = off;
  off = align256(off + int64_t(p->row_a.size() * 4));
  L.row_b = off;
  off = align256(off + int64_t(p->row_b.size() * 4));
  L.mask = off;
  off = align256(off + int64_t(p->row_mask.size() * 8));
  L.merge = off;
  off = align256(off + int64_t(p->merge.size() * sizeof(MergeRow)));
  L.kwork = off;
  off = align256(off + int64_t(p->kwork.size() * sizeof(WorkItem)));
  L.kmerge = off;
  off = align256(off + int64_t(p->kmerge.size() * sizeof(KMerge)));
  L.trees = off;
  off = align256(off + int64_t(p->tree_tab.size() * 4));
  L.tile_a = off;
  off = align256(off + int64_t(p->tile_a.size() * 4));
  L.tile_b = off;
  off = align256(off + int64_t(p->tile_b.size() * 4));
  L.total = std::max<int64_t>(off, 256);
  // the image is built aside and swapped in, so a failed allocation leaves
  // the plan as it was
  std::vector<unsigned char> blob(size_t(L.total), 0);
  auto put = [&](int64_t at, const void* src, size_t n) {
    if (n) std::memcpy(blob.data() + at, src, n);
  };
  put(L.work, p->work.data(), p->work.size() * sizeof(WorkItem));
  put(L.row_a, p->row_a.data(), p->row_a.size() * 4);
  put(L.row_b, p->row_b.data(), p->row_b.size() * 4);
  put(L.mask, p->row_mask.data(), p->row_mask.size() * 8);
  put(L.merge, p->merge.data(), p->merge.size() * sizeof(MergeRow));
  put(L.kwork, p->kwork.data(), p->kwork.size() * sizeof(WorkItem));
  put(L.kmerge, p->kmerge.data(), p->kmerge.size() * sizeof(KMerge));
  put(L.trees, p->tree_tab.data(), p->tree_tab.size() * 4);
  put(L.tile_a, p->tile_a.data(), p->tile_a.size() * 4);
  put(L.tile_b, p->tile_b.data(), p->tile_b.size() * 4);
  p->blob.swap(blob);
  p->layout = L;
}

}  // namespace ta

using namespace ta;

extern "C" int tree_attn_plan_prefill(const int32_t* prefix_len, const int32_t* n_regions,
                                      const int32_t* layout_len, const int32_t* content_len,
                                      int32_t n_pages, ta_plan** out) try {
  if (!out) return fail(TA_ERR_INVALID_ARG, "plan_prefill: out is NULL");
  if (n_pages < 0) return fail(TA_ERR_INVALID_ARG, "plan_prefill: n_pages < 0");
  if (n_pages > 0 && (!prefix_len || !n_regions))
    return fail(TA_ERR_INVALID_ARG, "plan_prefill: NULL prefix_len/n_regions");
  int64_t total_regions = 0, total_tokens = 0;
  for (int32_t p = 0; p < n_pages; ++p) {
    if (prefix_len[p] < 0) return fail(TA_ERR_INVALID_ARG, "plan_prefill: negative prefix_len");
    if (n_regions[p] < 0) return fail(TA_ERR_INVALID_ARG, "plan_prefill: negative n_regions");
    total_regions += n_regions[p];
  }
  if (total_regions > 0 && (!layout_len || !content_len))
    return fail(TA_ERR_INVALID_ARG, "plan_prefill: NULL layout_len/content_len");
  for (int64_t r = 0; r < total_regions; ++r) {
    if (layout_len[r] < 0 || content_len[r] < 0)
      return fail(TA_ERR_INVALID_ARG, "plan_prefill: negative layout/content length");
  }
  {
    int64_t r = 0;
    for (int32_t p = 0; p < n_pages; ++p) {
      total_tokens += prefix_len[p];
      for (int32_t k = 0; k < n_regions[p]; ++k, ++r) total_tokens += int64_t(layout_len[r]) + content_len[r];
      if (total_tokens >= kMax32) return fail(TA_ERR_CAPACITY, "plan_prefill: packed length >= 2^31");
    }
  }

  // owned here until handed out, so a throwing resize cannot leak it
  std::unique_ptr<ta_plan> owner(new ta_plan());
  ta_plan* pl = owner.get();
  pl->kind = TA_PLAN_PREFILL;
  pl->n_pages = n_pages;
  pl->n_branches = int32_t(total_regions);
  pl->n_rows = total_tokens;
  pl->n_keys_a = pl->n_keys_b = total_tokens;
  pl->row_a.resize(size_t(total_tokens));
  pl->row_b.resize(size_t(total_tokens));
  pl->position.resize(size_t(total_tokens));
  pl->main_end.resize(size_t(total_tokens));
  pl->branch_start.resize(size_t(total_tokens));

  int64_t base = 0, r = 0;
  for (int32_t p = 0; p < n_pages; ++p) {
    const int64_t P = prefix_len[p];
    const int32_t N = n_regions[p];
    int64_t sumL = 0, sumC = 0;
    for (int32_t k = 0; k < N; ++k) {
      sumL += layout_len[r + k];
      sumC += content_len[r + k];
    }
    const int64_t M = P + sumL, T = M + sumC;
    // main stream: causal over [X | B]
    for (int64_t i = 0; i < M; ++i) {
      const int64_t row = base + i;
      pl->position[row] = i;
      pl->main_end[row] = row + 1;
      pl->branch_start[row] = row + 1;
    }
    // branches
    int64_t accL = 0, accC = 0, depth = 0;
    for (int32_t k = 0; k < N; ++k) {
      accL += layout_len[r + k];
      const int64_t ck = content_len[r + k];
      const int64_t b0 = base + M + accC;
      const int64_t bound = base + P + accL;
      pl->branches3.insert(pl->branches3.end(), {bound, b0, ck});
      for (int64_t t = 0; t < ck; ++t) {
        pl->position[b0 + t] = P + accL + t;
        pl->main_end[b0 + t] = bound;
        pl->branch_start[b0 + t] = b0;
      }
      accC += ck;
      depth = std::max(depth, accL + ck);
    }
    pl->pages5.insert(pl->pages5.end(), {base, M, T, depth, sumL + sumC});
    pl->max_depth = std::max(pl->max_depth, depth);
    for (int64_t i = 0; i < T; ++i) pl->visible_pairs += pl->position[base + i] + 1;

    // row tiles of this page
    for (int64_t t0 = 0; t0 < T; t0 += kTileTokens) {
      const int64_t t1 = std::min(T, t0 + kTileTokens);
      int64_t a_hi = base, a_full = INT64_MAX, b_lo = INT64_MAX, b_hi = 0;
      bool any_branch = false;
      for (int64_t i = base + t0; i < base + t1; ++i) {
        a_hi = std::max(a_hi, pl->main_end[i]);
        a_full = std::min(a_full, pl->main_end[i]);
        if (pl->branch_start[i] <= i) {
          any_branch = true;
          b_lo = std::min(b_lo, pl->branch_start[i]);
          b_hi = std::max(b_hi, i + 1);
        }
      }
      if (!any_branch) b_lo = b_hi = 0;
      // a main-stream row's own causal bound is inside segment A, so a tile
      // holding main rows is fully visible only below its first row.
      pl->work.push_back(make_item(base + t0, t1 - t0, base, a_full, a_hi, b_lo, b_hi, -1, 0));
    }

    // key-major tiles for the backward: a main key j is seen by the main rows
    // [j, M) and by the rows of every branch whose bound exceeds j (bounds
    // grow with k, so those rows form a suffix of the page); a branch key j
    // of Y_k by the rows [j, end of Y_k)
    std::vector<int64_t> bound(static_cast<size_t>(N)), bstart(static_cast<size_t>(N)), blen(static_cast<size_t>(N));
    {
      int64_t aL = 0, aC = 0;
      for (int32_t k = 0; k < N; ++k) {
        aL += layout_len[r + k];
        bound[k] = base + P + aL;
        bstart[k] = base + M + aC;
        blen[k] = content_len[r + k];
        aC += content_len[r + k];
      }
    }
    auto row_tiles = [](int64_t lo, int64_t hi) { return hi > lo ? (hi - lo + kKeyTile - 1) / kKeyTile : 0; };
    // one item per key tile, or near-equal pieces of its row tiles when the
    // walk is long (they write fp32 partials that a merge sums in order)
    auto push_key_item = [&](WorkItem w, int64_t n_rt) {
      const int64_t np = std::max<int64_t>(1, (n_rt + kBwdMaxRowTiles - 1) / kBwdMaxRowTiles);
      if (np > 1) pl->kmerge.push_back(KMerge{w.row0, w.nrows, int32_t(pl->n_kpart), int32_t(np)});
      for (int64_t i = 0; i < np; ++i) {
        w.tile_lo = int32_t(n_rt * i / np);
        w.tile_hi = int32_t(n_rt * (i + 1) / np);
        w.b_full = np > 1 ? int32_t(pl->n_kpart++) : -1;
        pl->kwork.push_back(w);
      }
    };
    for (int64_t k0 = base; k0 < base + M; k0 += kKeyTile) {
      const int64_t k1 = std::min(base + M, k0 + kKeyTile);
      int64_t first = base + T;  // first row of the first non-empty branch that sees key k0
      for (int32_t k = 0; k < N; ++k)
        if (bound[k] > k0 && blen[k] > 0) {
          first = bstart[k];
          break;
        }
      int64_t full_b = base + T;  // first row of the first non-empty branch that sees all of [k0, k1)
      for (int32_t k = 0; k < N; ++k)
        if (bound[k] >= k1 && blen[k] > 0) {
          full_b = bstart[k];
          break;
        }
      // main rows r >= k1 - 1 see every key of the tile; so do the rows of
      // every branch from full_b on
      push_key_item(make_item(k0, k1 - k0, k0, k1 - 1, base + M, first, base + T, std::max(full_b, first), 0),
                    row_tiles(k0, base + M) + row_tiles(first, base + T));
    }
    for (int64_t k0 = base + M; k0 < base + T; k0 += kKeyTile) {
      const int64_t k1 = std::min(base + T, k0 + kKeyTile);
      int64_t end = k1;  // end of the last branch with a key in [k0, k1)
      for (int32_t k = 0; k < N; ++k)
        if (bstart[k] < k1 && bstart[k] + blen[k] > k0) end = std::max(end, bstart[k] + blen[k]);
      push_key_item(make_item(k0, k1 - k0, k0, end, end, 0, 0, 0, kKeyBranch), row_tiles(k0, end));
    }
    base += T;
    r += N;
  }
  std::stable_sort(pl->kwork.begin(), pl->kwork.end(), [](const WorkItem& x, const WorkItem& y) {
    return x.tile_hi - x.tile_lo > y.tile_hi - y.tile_lo;
  });
  for (int64_t i = 0; i < total_tokens; ++i) {
    pl->row_a[i] = int32_t(pl->main_end[i]);
    pl->row_b[i] = int32_t(pl->branch_start[i]);
  }
  order_work_paged(pl->work, pl->pages5);
  pack_blob(pl);
  *out = owner.release();
  return TA_OK;
} catch (...) {
  return ta::fail_exception("plan_prefill");
}

namespace {

// Decode plan with n_query[b] new tokens per live branch (NULL: one each).
// With paging, the pages' main streams (pa, per page) and the branches'
// suffixes (pb, per branch) are read through block tables; their virtual
// positions start on 64-token boundaries.
int build_decode(const int32_t* prefix_len, const int32_t* n_regions, const int32_t* layout_len, int32_t n_pages,
                 const int32_t* br_page, const int32_t* br_region, const int32_t* suffix_len,
                 const int32_t* n_query, int32_t n_branches, const Paging& pa, const Paging& pb, ta_plan** out) {
  if (!out) return fail(TA_ERR_INVALID_ARG, "plan_decode: out is NULL");
  if (n_pages < 0 || n_branches < 0) return fail(TA_ERR_INVALID_ARG, "plan_decode: negative count");
  if (n_pages > 0 && (!prefix_len || !n_regions))
    return fail(TA_ERR_INVALID_ARG, "plan_decode: NULL prefix_len/n_regions");
  if (n_branches > 0 && (!br_page || !br_region || !suffix_len))
    return fail(TA_ERR_INVALID_ARG, "plan_decode: NULL branch arrays");
  std::vector<int64_t> reg_off(size_t(n_pages) + 1, 0), main_off(size_t(n_pages) + 1, 0);
  for (int32_t p = 0; p < n_pages; ++p) {
    if (prefix_len[p] < 0 || n_regions[p] < 0) return fail(TA_ERR_INVALID_ARG, "plan_decode: negative page size");
    reg_off[p + 1] = reg_off[p] + n_regions[p];
  }
  if (reg_off[n_pages] > 0 && !layout_len) return fail(TA_ERR_INVALID_ARG, "plan_decode: NULL layout_len");
  std::vector<int64_t> page_len(static_cast<size_t>(n_pages));
  for (int32_t p = 0; p < n_pages; ++p) {
    int64_t m = prefix_len[p];
    for (int64_t r = reg_off[p]; r < reg_off[p + 1]; ++r) {
      if (layout_len[r] < 0) return fail(TA_ERR_INVALID_ARG, "plan_decode: negative layout_len");
      m += layout_len[r];
    }
    page_len[p] = m;
    main_off[p + 1] = main_off[p] + (pa.on() ? round_tile(m) : m);
    if (main_off[p + 1] >= kMax32) return fail(TA_ERR_CAPACITY, "plan_decode: main tokens >= 2^31");
  }
  auto kq = [&](int32_t b) -> int64_t { return n_query ? n_query[b] : 1; };
  int64_t suffix_total = 0, rows_total = 0;
  for (int32_t b = 0; b < n_branches; ++b) {
    if (br_page[b] < 0 || br_page[b] >= n_pages) return fail(TA_ERR_INVALID_ARG, "plan_decode: br_page out of range");
    if (b > 0 && br_page[b] < br_page[b - 1])
      return fail(TA_ERR_INVALID_ARG, "plan_decode: branches must be grouped by page (br_page non-decreasing)");
    if (br_region[b] < 0 || br_region[b] > n_regions[br_page[b]])
      return fail(TA_ERR_INVALID_ARG, "plan_decode: br_region must be 0 (layout stream) or 1..N of its page");
    if (suffix_len[b] < 0) return fail(TA_ERR_INVALID_ARG, "plan_decode: negative suffix_len");
    if (kq(b) < 1) return fail(TA_ERR_INVALID_ARG, "plan_decode: n_query must be >= 1");
    suffix_total += pb.on() ? round_tile(int64_t(suffix_len[b]) + kq(b)) : int64_t(suffix_len[b]) + kq(b);
    rows_total += kq(b);
    if (suffix_total >= kMax32) return fail(TA_ERR_CAPACITY, "plan_decode: suffix tokens >= 2^31");
    if (rows_total >= kMax32) return fail(TA_ERR_CAPACITY, "plan_decode: query rows >= 2^31");
  }

  std::vector<int64_t> suf_len(static_cast<size_t>(n_branches));
  for (int32_t b = 0; b < n_branches; ++b) suf_len[b] = int64_t(suffix_len[b]) + kq(b);
  if (pa.on()) {
    int rc = check_paging(pa, n_pages, page_len, "plan_decode_paged (main)");
    if (!rc) rc = check_paging(pb, n_branches, suf_len, "plan_decode_paged (suffix)");
    if (rc) return rc;
  }

  // owned here until handed out, so a throwing resize cannot leak it
  std::unique_ptr<ta_plan> owner(new ta_plan());
  ta_plan* pl = owner.get();
  pl->kind = TA_PLAN_DECODE;
  pl->n_pages = n_pages;
  pl->n_branches = n_branches;
  pl->n_rows = rows_total;
  pl->n_keys_a = pa.on() ? int64_t(pa.n_cache_blocks) * pa.bs : main_off[n_pages];
  pl->n_keys_b = pb.on() ? int64_t(pb.n_cache_blocks) * pb.bs : suffix_total;
  pl->row_a.resize(size_t(rows_total));
  pl->row_b.resize(size_t(rows_total));
  pl->merge.resize(size_t(rows_total));

  // per row: main bound (page-relative); per branch: first row, suffix start
  std::vector<int64_t> main_len(static_cast<size_t>(rows_total));
  std::vector<int64_t> row_off(static_cast<size_t>(n_branches) + 1, 0), suf_start(static_cast<size_t>(n_branches));
  int64_t s0 = 0;
  for (int32_t b = 0; b < n_branches; ++b) {
    const int32_t p = br_page[b];
    const int32_t n_reg = br_region[b] > 0 ? br_region[b] : n_regions[p];  // layout stream: all of B
    int64_t m = prefix_len[p];
    for (int32_t k = 0; k < n_reg; ++k) m += layout_len[reg_off[p] + k];
    suf_start[b] = s0;
    row_off[b + 1] = row_off[b] + kq(b);
    for (int64_t j = 0; j < kq(b); ++j) {
      const int64_t r = row_off[b] + j;
      const int64_t vis_suffix = int64_t(suffix_len[b]) + j + 1;
      main_len[r] = m;
      pl->row_a[r] = int32_t(main_off[p] + m);
      pl->row_b[r] = int32_t(s0 + vis_suffix);
      pl->decode_rows5.insert(pl->decode_rows5.end(), {main_off[p], m, s0, vis_suffix, m + vis_suffix - 1});
      pl->visible_pairs += m + vis_suffix;
    }
    s0 += pb.on() ? round_tile(suf_len[b]) : suf_len[b];
  }
  if (pa.on()) {
    fill_tiles(pa, n_pages, page_len, main_off, main_off[n_pages], pl->tile_a);
    fill_tiles(pb, n_branches, suf_len, suf_start, suffix_total, pl->tile_b);
  }

  // Chunk length: the longest (down to kDecodeChunkMin) that keeps at least
  // kDecodeMinItems pass-1 items.
  auto n_items = [&](int64_t chunk) {
    int64_t n = 0;
    for (int32_t b0 = 0, e0; b0 < n_branches; b0 = e0) {
      e0 = b0;
      while (e0 < n_branches && br_page[e0] == br_page[b0]) ++e0;
      for (int64_t g0 = row_off[b0]; g0 < row_off[e0]; g0 += kTileTokens) {
        int64_t hi = 0;
        for (int64_t i = g0; i < std::min(row_off[e0], g0 + kTileTokens); ++i) hi = std::max(hi, main_len[i]);
        n += (hi + chunk - 1) / chunk;
      }
    }
    for (int32_t i = 0; i < n_branches; ++i)
      for (int64_t j0 = 0; j0 < kq(i); j0 += kTileTokens) {
        const int64_t len = int64_t(suffix_len[i]) + std::min(kq(i), j0 + kTileTokens);
        n += len <= kDecodeSuffixWhole ? 1 : (len + chunk - 1) / chunk;
      }
    return n;
  };
  int64_t dchunk = kDecodeChunkMax;
  while (dchunk > kDecodeChunkMin && n_items(dchunk) < kDecodeMinItems) dchunk /= 2;

  // Pass-1 work items.  Partial slots (per query head) are numbered in plan
  // order: a shared chunk owns one slot per row of its row group, and so does
  // a suffix chunk.
  int64_t slot = 0;
  int32_t b = 0;
  while (b < n_branches) {
    const int32_t p = br_page[b];
    int32_t e = b;
    while (e < n_branches && br_page[e] == p) ++e;
    // row groups of at most one tile of the page's rows; with more than one
    // group, every group walks the page's main stream
    const int32_t a_shared = row_off[e] - row_off[b] > kTileTokens ? kSegAShared : 0;
    for (int64_t g0 = row_off[b]; g0 < row_off[e]; g0 += kTileTokens) {
      const int64_t g1 = std::min(row_off[e], g0 + kTileTokens);
      int64_t hi = 0, lo_bound = INT64_MAX;
      for (int64_t i = g0; i < g1; ++i) {
        hi = std::max(hi, main_len[i]);
        lo_bound = std::min(lo_bound, main_len[i]);
      }
      const int64_t n_chunks = (hi + dchunk - 1) / dchunk;
      const int64_t first = slot;
      for (int64_t c = 0; c < n_chunks; ++c) {
        const int64_t c0 = c * dchunk, c1 = std::min(hi, c0 + dchunk);
        pl->work.push_back(make_item(g0, g1 - g0, main_off[p] + c0, main_off[p] + lo_bound, main_off[p] + c1,
                                     0, 0, slot, a_shared));
        slot += g1 - g0;
      }
      for (int64_t i = g0; i < g1; ++i) {
        MergeRow& mr = pl->merge[i];
        mr.row = int32_t(i);
        mr.sh_first = int32_t(first + (i - g0));
        mr.sh_count = int32_t((main_len[i] + dchunk - 1) / dchunk);
        mr.sh_stride = int32_t(g1 - g0);
      }
    }
    b = e;
  }
  // Suffix items: per branch, row groups of at most one tile of its new
  // tokens; row j of the branch sees suffix keys [start, start + s + j + 1).
  for (int32_t i = 0; i < n_branches; ++i) {
    const int64_t s = suffix_len[i];
    for (int64_t j0 = 0; j0 < kq(i); j0 += kTileTokens) {
      const int64_t j1 = std::min(kq(i), j0 + kTileTokens);
      const int64_t len = s + j1;             // keys the group's last row sees
      const int64_t full = suf_start[i] + s + j0 + 1;  // keys every row of the group sees end here
      const int64_t chunk = len <= kDecodeSuffixWhole ? len : dchunk;
      const int64_t n_chunks = (len + chunk - 1) / chunk;
      const int64_t first = slot;
      for (int64_t c = 0; c < n_chunks; ++c) {
        const int64_t c0 = suf_start[i] + c * chunk, c1 = std::min(suf_start[i] + len, c0 + chunk);
        const int32_t flags = (c1 <= full ? kSegBFull : 0) | (kq(i) > kTileTokens ? kSegBShared : 0);
        WorkItem w = make_item(row_off[i] + j0, j1 - j0, 0, 0, 0, c0, c1, slot, flags);
        w.b_full = int32_t(std::max(c0, std::min(c1, full)));
        pl->work.push_back(w);
        slot += j1 - j0;
      }
      for (int64_t j = j0; j < j1; ++j) {
        MergeRow& mr = pl->merge[row_off[i] + j];
        mr.sf_first = int32_t(first + (j - j0));
        mr.sf_count = int32_t((s + j + 1 + chunk - 1) / chunk);
        mr.sf_stride = int32_t(j1 - j0);
      }
    }
  }
  if (slot >= kMax32) {
    return fail(TA_ERR_CAPACITY, "plan_decode: partial slots >= 2^31");
  }
  pl->n_partials = slot;
  order_work(pl->work);
  pack_blob(pl);
  *out = owner.release();
  return TA_OK;
}

}  // namespace

extern "C" int tree_attn_plan_decode(const int32_t* prefix_len, const int32_t* n_regions,
                                     const int32_t* layout_len, int32_t n_pages,
                                     const int32_t* br_page, const int32_t* br_region,
                                     const int32_t* suffix_len, int32_t n_branches,
                                     ta_plan** out) try {
  return build_decode(prefix_len, n_regions, layout_len, n_pages, br_page, br_region, suffix_len, nullptr,
                      n_branches, Paging{}, Paging{}, out);
} catch (...) {
  return ta::fail_exception("plan_decode");
}

extern "C" int tree_attn_plan_decode_multi(const int32_t* prefix_len, const int32_t* n_regions,
                                           const int32_t* layout_len, int32_t n_pages,
                                           const int32_t* br_page, const int32_t* br_region,
                                           const int32_t* suffix_len, const int32_t* n_query,
                                           int32_t n_branches, ta_plan** out) try {
  if (n_branches > 0 && !n_query) return fail(TA_ERR_INVALID_ARG, "plan_decode_multi: NULL n_query");
  return build_decode(prefix_len, n_regions, layout_len, n_pages, br_page, br_region, suffix_len, n_query,
                      n_branches, Paging{}, Paging{}, out);
} catch (...) {
  return ta::fail_exception("plan_decode_multi");
}

extern "C" int tree_attn_plan_decode_paged(const int32_t* prefix_len, const int32_t* n_regions,
                                           const int32_t* layout_len, int32_t n_pages,
                                           const int32_t* br_page, const int32_t* br_region,
                                           const int32_t* suffix_len, const int32_t* n_query,
                                           int32_t n_branches, int32_t block_size, int32_t n_cache_blocks,
                                           const int32_t* main_blocks, const int64_t* main_block_off,
                                           const int32_t* suffix_blocks, const int64_t* suffix_block_off,
                                           ta_plan** out) try {
  Paging pa, pb;
  pa.bs = pb.bs = block_size;
  pa.n_cache_blocks = pb.n_cache_blocks = n_cache_blocks;
  pa.blocks = main_blocks;
  pa.off = main_block_off;
  pb.blocks = suffix_blocks;
  pb.off = suffix_block_off;
  if (block_size <= 0) return fail(TA_ERR_INVALID_ARG, "plan_decode_paged: block_size must be a positive multiple of 64");
  return build_decode(prefix_len, n_regions, layout_len, n_pages, br_page, br_region, suffix_len, n_query,
                      n_branches, pa, pb, out);
} catch (...) {
  return ta::fail_exception("plan_decode_paged");
}

namespace {

// Verify plan; with paging the pages' contexts are read through block tables
// (virtual positions on 64-token boundaries) and tree nodes stay contiguous.
int build_verify(const int32_t* ctx_len, int32_t n_pages, const int32_t* br_page, const int32_t* n_nodes,
                 const int32_t* parent, int32_t n_branches, const Paging& pa, ta_plan** out) {
  if (!out) return fail(TA_ERR_INVALID_ARG, "plan_verify: out is NULL");
  if (n_pages < 0 || n_branches < 0) return fail(TA_ERR_INVALID_ARG, "plan_verify: negative count");
  if (n_pages > 0 && !ctx_len) return fail(TA_ERR_INVALID_ARG, "plan_verify: NULL ctx_len");
  if (n_branches > 0 && (!br_page || !n_nodes)) return fail(TA_ERR_INVALID_ARG, "plan_verify: NULL branch arrays");
  std::vector<int64_t> ctx_off(size_t(n_pages) + 1, 0);
  for (int32_t p = 0; p < n_pages; ++p) {
    if (ctx_len[p] < 0) return fail(TA_ERR_INVALID_ARG, "plan_verify: negative ctx_len");
    ctx_off[p + 1] = ctx_off[p] + (pa.on() ? round_tile(ctx_len[p]) : ctx_len[p]);
    if (ctx_off[p + 1] >= kMax32) return fail(TA_ERR_CAPACITY, "plan_verify: context tokens >= 2^31");
  }
  int64_t total_nodes = 0;
  for (int32_t b = 0; b < n_branches; ++b) {
    if (br_page[b] < 0 || br_page[b] >= n_pages) return fail(TA_ERR_INVALID_ARG, "plan_verify: br_page out of range");
    if (b > 0 && br_page[b] < br_page[b - 1])
      return fail(TA_ERR_INVALID_ARG, "plan_verify: trees must be grouped by page (br_page non-decreasing)");
    if (n_nodes[b] < 0) return fail(TA_ERR_INVALID_ARG, "plan_verify: negative n_nodes");
    if (n_nodes[b] > 64) return fail(TA_ERR_CAPACITY, "plan_verify: a tree has more than 64 nodes");
    total_nodes += n_nodes[b];
    if (total_nodes >= kMax32) return fail(TA_ERR_CAPACITY, "plan_verify: nodes >= 2^31");
  }
  if (total_nodes > 0 && !parent) return fail(TA_ERR_INVALID_ARG, "plan_verify: NULL parent");
  {
    int64_t off = 0;
    for (int32_t b = 0; b < n_branches; ++b) {
      for (int32_t i = 0; i < n_nodes[b]; ++i) {
        const int32_t pa = parent[off + i];
        if (pa < -1 || pa >= i)
          return fail(TA_ERR_INVALID_ARG, "plan_verify: parent must be -1 or an earlier node of the same tree");
      }
      off += n_nodes[b];
    }
  }

  std::vector<int64_t> clen(static_cast<size_t>(n_pages));
  for (int32_t p = 0; p < n_pages; ++p) clen[p] = ctx_len[p];
  if (pa.on()) {
    const int rc = check_paging(pa, n_pages, clen, "plan_verify_paged");
    if (rc) return rc;
  }

  // owned here until handed out, so a throwing resize cannot leak it
  std::unique_ptr<ta_plan> owner(new ta_plan());
  ta_plan* pl = owner.get();
  pl->kind = TA_PLAN_VERIFY;
  pl->n_pages = n_pages;
  pl->n_branches = n_branches;
  pl->n_rows = total_nodes;
  pl->n_keys_a = pa.on() ? int64_t(pa.n_cache_blocks) * pa.bs : ctx_off[n_pages];
  pl->n_keys_b = total_nodes;
  if (pa.on()) fill_tiles(pa, n_pages, clen, ctx_off, ctx_off[n_pages], pl->tile_a);
  pl->row_a.resize(size_t(total_nodes));
  pl->row_b.resize(size_t(total_nodes));
  pl->row_mask.resize(size_t(total_nodes));
  pl->verify_mask.resize(size_t(total_nodes));

  std::vector<int64_t> node_off(size_t(n_branches) + 1, 0);
  for (int32_t b = 0; b < n_branches; ++b) node_off[b + 1] = node_off[b] + n_nodes[b];
  pl->tree_tab.reserve(size_t(n_branches) + 1 + size_t(total_nodes));
  for (int32_t b = 0; b <= n_branches; ++b) pl->tree_tab.push_back(int32_t(node_off[b]));
  pl->tree_tab.insert(pl->tree_tab.end(), parent, parent + total_nodes);
  for (int32_t b = 0; b < n_branches; ++b) {
    const int32_t p = br_page[b];
    std::vector<uint64_t> bits(static_cast<size_t>(n_nodes[b]));
    std::vector<int64_t> dep(static_cast<size_t>(n_nodes[b]));
    for (int32_t i = 0; i < n_nodes[b]; ++i) {
      const int32_t pa = parent[node_off[b] + i];
      bits[i] = (pa < 0 ? 0ull : bits[pa]) | (1ull << i);
      dep[i] = pa < 0 ? 0 : dep[pa] + 1;
      const int64_t row = node_off[b] + i;
      pl->row_a[row] = int32_t(ctx_off[p] + ctx_len[p]);
      pl->row_b[row] = int32_t(node_off[b]);
      pl->row_mask[row] = bits[i];
      pl->verify_mask[row] = int64_t(bits[i]);
      pl->verify_rows4.insert(pl->verify_rows4.end(), {ctx_off[p], int64_t(ctx_len[p]), node_off[b], ctx_len[p] + dep[i]});
      pl->visible_pairs += ctx_len[p] + dep[i] + 1;
      pl->max_depth = std::max(pl->max_depth, dep[i]);
    }
  }
  // Row tiles: whole trees of one page, at most one tile of nodes.
  int32_t b = 0;
  while (b < n_branches) {
    const int32_t p = br_page[b];
    int32_t e = b;
    int64_t nodes = 0;
    while (e < n_branches && br_page[e] == p && nodes + n_nodes[e] <= kTileTokens) nodes += n_nodes[e++];
    if (nodes > 0) {
      pl->work.push_back(make_item(node_off[b], nodes, ctx_off[p], ctx_off[p] + ctx_len[p], ctx_off[p] + ctx_len[p],
                                   node_off[b], node_off[e], -1, 0));
    }
    b = e;
  }
  order_work(pl->work);
  pack_blob(pl);
  *out = owner.release();
  return TA_OK;
}

}  // namespace

extern "C" int tree_attn_plan_verify(const int32_t* ctx_len, int32_t n_pages, const int32_t* br_page,
                                     const int32_t* n_nodes, const int32_t* parent, int32_t n_branches,
                                     ta_plan** out) try {
  return build_verify(ctx_len, n_pages, br_page, n_nodes, parent, n_branches, Paging{}, out);
} catch (...) {
  return ta::fail_exception("plan_verify");
}

extern "C" int tree_attn_plan_verify_paged(const int32_t* ctx_len, int32_t n_pages, const int32_t* br_page,
                                           const int32_t* n_nodes, const int32_t* parent, int32_t n_branches,
                                           int32_t block_size, int32_t n_cache_blocks, const int32_t* ctx_blocks,
                                           const int64_t* ctx_block_off, ta_plan** out) try {
  Paging pa;
  pa.bs = block_size;
  pa.n_cache_blocks = n_cache_blocks;
  pa.blocks = ctx_blocks;
  pa.off = ctx_block_off;
  if (block_size <= 0) return fail(TA_ERR_INVALID_ARG, "plan_verify_paged: block_size must be a positive multiple of 64");
  return build_verify(ctx_len, n_pages, br_page, n_nodes, parent, n_branches, pa, out);
} catch (...) {
  return ta::fail_exception("plan_verify_paged");
}

namespace {

// Makespan of dispatching `jobs` (costs, in dispatch order, each once per KV
// head with the heads adjacent) to `slots` identical workgroup slots, each
// job going to the slot that frees first.
int64_t simulate_makespan(const std::vector<int64_t>& jobs, int hkv, int slots) {
  std::vector<int64_t> heap(size_t(slots), 0);  // min-heap of slot finish times
  auto cmp = [](int64_t a, int64_t b) { return a > b; };
  for (int64_t c : jobs)
    for (int k = 0; k < hkv; ++k) {
      std::pop_heap(heap.begin(), heap.end(), cmp);
      heap.back() += c;
      std::push_heap(heap.begin(), heap.end(), cmp);
    }
  return *std::max_element(heap.begin(), heap.end());
}

constexpr int64_t kItemOverhead = 3;  // prologue/epilogue of a workgroup, in tiles

}  // namespace

extern "C" int tree_attn_plan_balance(ta_plan* plan, int32_t n_kv_heads, int32_t n_slots) try {
  if (!plan) return fail(TA_ERR_INVALID_ARG, "plan_balance: plan is NULL");
  if (n_kv_heads <= 0 || n_slots <= 0) return fail(TA_ERR_INVALID_ARG, "plan_balance: counts must be positive");
  if (plan->kind == TA_PLAN_DECODE) return TA_OK;  // decode items are already key chunks
  if (plan->dev) return fail(TA_ERR_STATE, "plan_balance: plan already uploaded");
  if (plan->n_partials > 0) return fail(TA_ERR_STATE, "plan_balance: plan already balanced");
  // pieces as (item, tile_lo, tile_hi)
  struct Piece { int32_t item, lo, hi; };
  std::vector<WorkItem>& work = plan->work;
  std::vector<Piece> pieces;
  int64_t total = 0;
  for (int32_t i = 0; i < int32_t(work.size()); ++i) {
    pieces.push_back({i, 0, work[i].tile_hi});
    total += work[i].tile_hi + kItemOverhead;
  }
  auto cost = [](const Piece& p) { return int64_t(p.hi - p.lo) + kItemOverhead; };
  auto order = [&](std::vector<Piece>& v) {
    std::stable_sort(v.begin(), v.end(), [&](const Piece& a, const Piece& b) { return cost(a) > cost(b); });
  };
  const double balanced = double(total) * n_kv_heads / n_slots;
  for (int iter = 0; iter < 1024 && !pieces.empty(); ++iter) {
    order(pieces);
    std::vector<int64_t> jobs;
    for (const Piece& p : pieces) jobs.push_back(cost(p));
    const int64_t mk = simulate_makespan(jobs, n_kv_heads, n_slots);
    if (double(mk) <= 1.08 * balanced + kItemOverhead) break;
    Piece& big = pieces.front();
    if (big.hi - big.lo < 4) break;  // not worth splitting further
    const int32_t mid = big.lo + (big.hi - big.lo) / 2;
    Piece tail{big.item, mid, big.hi};
    big.hi = mid;
    pieces.push_back(tail);
  }
  // Rebuild the work list: unsplit items stay direct; the pieces of a split
  // item get consecutive partial slots (piece p, row t -> base + p*nrows + t).
  std::vector<int32_t> n_pieces(work.size(), 0);
  for (const Piece& p : pieces) n_pieces[p.item]++;
  std::sort(pieces.begin(), pieces.end(),
            [](const Piece& a, const Piece& b) { return a.item != b.item ? a.item < b.item : a.lo < b.lo; });
  std::vector<WorkItem> out;
  std::vector<MergeRow> merge;
  int64_t slot = 0;
  size_t k = 0;
  while (k < pieces.size()) {
    const int32_t item = pieces[k].item;
    const WorkItem& w = work[item];
    if (n_pieces[item] == 1) {
      out.push_back(w);
      ++k;
      continue;
    }
    const int64_t base = slot;
    for (int32_t pc = 0; pc < n_pieces[item]; ++pc, ++k) {
      WorkItem piece = w;
      piece.tile_lo = pieces[k].lo;
      piece.tile_hi = pieces[k].hi;
      piece.out = int32_t(base + int64_t(pc) * w.nrows);
      out.push_back(piece);
    }
    for (int32_t t = 0; t < w.nrows; ++t) {
      MergeRow mr{};
      mr.sh_first = int32_t(base + t);
      mr.sh_count = n_pieces[item];
      mr.sh_stride = w.nrows;
      mr.sf_first = 0;
      mr.sf_count = 0;
      mr.sf_stride = 1;
      mr.row = w.row0 + t;
      merge.push_back(mr);
    }
    slot += int64_t(n_pieces[item]) * w.nrows;
    if (slot >= kMax32) return fail(TA_ERR_CAPACITY, "plan_balance: partial slots >= 2^31");
  }
  if (plan->kind == TA_PLAN_PREFILL) order_work_paged(out, plan->pages5);
  else order_work(out);
  plan->work.swap(out);
  plan->merge.swap(merge);
  const int64_t old_partials = plan->n_partials;
  plan->n_partials = slot;
  try {
    pack_blob(plan);
  } catch (...) {  // a failed balance leaves the plan unbalanced and usable
    plan->work.swap(out);
    plan->merge.swap(merge);
    plan->n_partials = old_partials;
    throw;
  }
  return TA_OK;
} catch (...) {
  return ta::fail_exception("plan_balance");
}
