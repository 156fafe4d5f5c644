// Internal definitions shared by the plan builder, the C ABI and the kernel
// launchers of libtree_attn.  Not part of the public interface.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/tree_attn.h"

namespace ta {

// Every launch walks row tiles of this many query tokens.
constexpr int kTileTokens = 64;
// Keys per LDS tile.
constexpr int kKeyTile = 64;
// Decode splits a page's main stream (and long suffixes) into chunks; each
// chunk is one work item producing fp32 partials.  Chunks are as long as
// possible (fewer partials to write and merge) while the launch keeps at
// least kDecodeMinItems items: the longest chunk that achieves that, halving
// from kDecodeChunkMax down to kDecodeChunkMin.
constexpr int kDecodeChunkMax = 8192;
constexpr int kDecodeChunkMin = 1024;
constexpr int kDecodeMinItems = 256;
// Suffixes up to this length stay in one work item.
constexpr int kDecodeSuffixWhole = 2048;

// One work item: a tile of query rows and the two key segments it walks.
//   rows  [row0, row0 + nrows)
//   seg A [a_lo, a_hi): keys [a_lo, a_full) are visible to every row of the
//         tile; keys in [a_full, a_hi) are tested per row against row_a.
//   seg B [b_lo, b_hi): tested per row (prefill: branch-causal; verify:
//         tree bitmask; decode suffix: key < row_b, so keys [b_lo, b_full)
//         are visible to every row of the tile and flag kSegBFull marks a
//         segment visible to all of them).
//   out   first partial slot of the tile (per query head) when the item
//         writes fp32 partials (decode; split prefill/verify pieces); else -1.
//   flags bit 0: seg B fully visible; bits 2 and 3 (decode): seg A / seg B
//         is also read by other items (several row groups of a page or of a
//         branch), so its copies keep the default cache policy instead of
//         streaming past the caches.
//   [tile_lo, tile_hi) the 64-key tiles (segment A's, then segment B's) this
//         item walks; a prefill/verify row tile split for load balance has
//         one item per piece.
struct WorkItem {
  int32_t row0, nrows, a_lo, a_full, a_hi, b_lo, b_hi, out;
  int32_t flags, tile_lo, tile_hi, b_full;
};
static_assert(sizeof(WorkItem) == 48, "work item layout");
constexpr int32_t kSegBFull = 1;
constexpr int32_t kSegAShared = 4;
constexpr int32_t kSegBShared = 8;
// Key-major work items of the prefill backward (dK, dV) reuse WorkItem:
//   keys  [row0, row0 + nrows) one 64-key tile of a page's main stream or
//         of its branch area; flags bit 1 set for the branch area
//   rows  [a_lo, a_hi) and [b_lo, b_hi): the query rows that can see a key
//         of the tile; rows from a_full (segment A) and from `out` (segment
//         B) on see every key of it.  Other row tiles are tested per row
//         against row_a / row_b: a main key is visible to rows with
//         key < row_a, a branch key to rows with row_b <= key <= row
//   [tile_lo, tile_hi) the item's 64-row tiles (segment A's, then B's) that
//         this piece walks; an item whose walk is longer than
//         kBwdMaxRowTiles is split into near-equal pieces
//   b_full  partial slot of a split piece (it writes fp32 dK, dV there), or
//         -1 when the piece is the whole item (it writes dK, dV directly)
constexpr int32_t kKeyBranch = 2;
constexpr int64_t kBwdMaxRowTiles = 100;

// A split key tile of the backward: keys [key0, key0 + nkeys) of every KV
// head sum the fp32 partials of slots [first, first + count), in slot order.
struct KMerge {
  int32_t key0, nkeys, first, count;
};
static_assert(sizeof(KMerge) == 16, "key merge layout");

// Merge table, one entry per output row combined from partials: slots are
// sh_first + c * sh_stride (c < sh_count), then sf_first + c * sf_stride
// (c < sf_count), merged in that order.  Decode: every branch (main-stream chunks, then its
// suffix chunks).  Prefill/verify: the rows of split row tiles.
struct MergeRow {
  int32_t sh_first, sh_count, sh_stride, sf_first, sf_count, row, sf_stride, pad0;
};
static_assert(sizeof(MergeRow) == 32, "merge row layout");

// Offsets (bytes) of the tables inside the device workspace.
struct DeviceLayout {
  int64_t work = 0, row_a = 0, row_b = 0, mask = 0, merge = 0, kwork = 0, kmerge = 0, trees = 0, tile_a = 0,
          tile_b = 0, total = 0;
};

}  // namespace ta

struct ta_plan {
  int32_t kind = 0;
  int32_t n_pages = 0;
  int32_t n_branches = 0;
  int64_t n_rows = 0;
  int64_t n_keys_a = 0;
  int64_t n_keys_b = 0;
  int64_t n_partials = 0;
  int64_t visible_pairs = 0;
  int64_t max_depth = 0;

  // device tables (host copies)
  std::vector<ta::WorkItem> work;
  std::vector<int32_t> row_a, row_b;
  std::vector<uint64_t> row_mask;
  std::vector<ta::MergeRow> merge;
  std::vector<ta::WorkItem> kwork;  // prefill: key-major items of the backward
  std::vector<ta::KMerge> kmerge;   // prefill: key tiles whose backward walk is split
  int64_t n_kpart = 0;              // partial slots of the split key tiles
  std::vector<int32_t> tree_tab;    // verify: node offsets [n_branches + 1], then parents [n_rows]
  // paged plans: physical cache row of the first token of every 64-token
  // tile of segment A / segment B, indexed by virtual position / 64 (empty
  // when that segment is contiguous)
  std::vector<int32_t> tile_a, tile_b;
  ta::DeviceLayout layout;
  std::vector<unsigned char> blob;  // packed image of the device tables

  // exported semantic fields
  std::vector<int64_t> position, main_end, branch_start, pages5, branches3;
  std::vector<int64_t> decode_rows5, verify_rows4, verify_mask;

  // binding to device memory
  void* dev = nullptr;
  void* upload_event = nullptr;  // hipEvent_t of the last upload
};

namespace ta {
int64_t item_tiles(const WorkItem& w);
void set_error(const std::string& msg);
int fail(int code, const std::string& msg);
int fail_exception(const char* who) noexcept;
void pack_blob(ta_plan* p);
}  // namespace ta
