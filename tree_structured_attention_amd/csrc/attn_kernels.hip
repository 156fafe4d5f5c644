// HIP kernels for layout-grounded tree attention on gfx950 (MI355X).
//
// One kernel template serves the three entry points.  A workgroup takes one
// work item (a tile of up to 64 query tokens, times the query heads of one
// KV head that it owns) and walks two key segments tile by tile:
//   prefill  seg A = the page's main stream [X | B] (per-row upper bound),
//            seg B = the content branches overlapping the tile (per-row
//            branch-causal interval)         -- PaDoc summary, "Training
//            paradigm": branch Y_k attends [X, B_<=k, Y_k]
//   verify   seg A = the page's accepted context (all visible),
//            seg B = the tile's draft-tree nodes (per-row ancestor bitmask)
//                                            -- HSD notes, key design 3 (b)
//   decode   seg A = one chunk of a page's main stream, shared by every live
//            branch and query head of the page (per-row bound P + L_<=k), or
//            seg B = one chunk of one branch's own suffix; the kernel writes
//            fp32 partials that a second kernel merges by log-sum-exp
//                                            -- PaDoc summary, "Inference";
//            HPD-Parsing notes, shared-prefix KV reuse
//
// MFMA formulation (wave64, one wave = 32 query rows):
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = Q
//   held in registers, so each lane owns one query row (lane % 32) and the
//   row's softmax statistics live in two lanes (lane, lane + 32).
//   O^T += V^T P^T: A = V^T read from a transposed LDS tile, B = P^T taken
//   straight from the S^T accumulators, so P never leaves registers.
//   K rows are loaded in a permuted order (bits 2 and 3 of the MFMA row index
//   swapped) so that the 8 keys a lane holds for the PV step are contiguous.
// Softmax is online in fp32 with exp2 and the scale folded into one FMA; the
// running rescale is skipped when no row of the wave raised its maximum.
// Non-visible scores are replaced by -inf (selection), padded keys are
// zero-filled, so no value outside a row's ancestors can reach its output
// unless it is a non-finite V of a key another row of the same tile needs.
// fp32 inputs use v_mfma_f32_32x32x2f32 with the same tiling (no
// down-conversion).
#include <mutex>

#include "ta_device.h"

namespace ta {

// Per-lane state of one wave: its 32 query rows (lane % 32) and the running
// softmax of each.
template <typename T, int D, int MODE>
struct RowState {
  static constexpr bool kBf = std::is_same<T, __bf16>::value;
  static constexpr int kQSteps = kBf ? D / 16 : D / 2;  // MFMA k-steps over head_dim
  static constexpr int kDB = D / 32;                    // 32-wide blocks of head_dim
  using G = TileGeom<T, D>;
  using QFrag = typename std::conditional<kBf, bf16x8, float>::type;

  QFrag qf[kQSteps];
  f32x16 acc[kDB];
  float m_used;  // exp2 base in raw-score units: a maximum of the scores so far (bf16: may lag the current one)
  float mbc;     // bf16: the exp2 offset m_used * c (0 while the base is unset), kept beside m_used
  bool unset;    // wave-uniform: some row of the wave has no base yet (bases never return to unset)
  float l_run;   // this lane's half of the row sum
  int koff[kBf ? kQSteps : 1];
  int voff[kBf ? 2 * kDB : 1];
  int h, n, lane_id, row, ra, rb;
  uint64_t rmask;
  bool row_ok;
  float c, tau;  // scale * log2(e); fp32: base move threshold

  __device__ __forceinline__ void init_offsets(int lane) {
    if constexpr (kBf) {
      const int krow0 = key_perm(n);
#pragma unroll
      for (int st = 0; st < kQSteps; ++st) koff[st] = G::at(krow0, D * h + 16 * st);
      const int m16 = lane & 15, grp = lane >> 4;
      // transposing reads: lane m of each 16-lane group addresses
      // V[key0 + m/4][d0 + 4 (m%4)]; lane i receives keys key0..key0+3 at d0 + i.
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int md = 0; md < kDB; ++md) {
          const int key = 8 * (grp >> 1) + 4 * r + (m16 >> 2);
          const int dbyte = 2 * (32 * md + 16 * (grp & 1) + 4 * (m16 & 3));
          voff[r * kDB + md] = G::at(key, dbyte);
        }
    }
  }

  // One 64-key tile from LDS (K at kl, V at vl).
  __device__ __forceinline__ void consume(const unsigned char* kl, const unsigned char* vl, int t0, int t_hi,
                                          bool seg_a, bool masked) {
    // ---- S^T = K Q^T for two 32-key blocks (interleaved chains) ----
    f32x16 s[2];
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[bk][i] = 0.f;
    if constexpr (kBf) {
      // the lane's K-row offsets of all k-steps stay in registers (computed
      // once per work item): no address arithmetic per tile
#pragma unroll
      for (int st = 0; st < kQSteps; ++st)
#pragma unroll
        for (int bk = 0; bk < 2; ++bk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kl + koff[st] + 32 * bk * G::kRowBytes);
          s[bk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[bk], 0, 0, 0);
        }
      sched_ld_mfma<0, 2 * kQSteps, 1, 4>();
    } else {
      const int krow0 = key_perm(n);
#pragma unroll
      for (int st = 0; st < kQSteps; ++st)
#pragma unroll
        for (int bk = 0; bk < 2; ++bk) {
          const float a = *reinterpret_cast<const float*>(kl + G::at(32 * bk + krow0, ((D / 2) * h + st) * 4));
          s[bk] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf[st], s[bk], 0, 0, 0);
        }
    }

    // ---- visibility: selection to -inf, only on tiles that need it ----
    if (masked) {
      // the row's visible keys of this tile, [lo, hi) and (verify, tree
      // segment) its ancestor bits, as one mask over the lane's key offsets;
      // a row past the item's end keeps every key below t_hi
      const int base = t0 + 8 * h;
      int lo = base, hi = t_hi;
      uint64_t tree = ~0ull;
      if (seg_a) {
        if constexpr (MODE != kVerify) hi = row_ok ? min(hi, ra) : hi;
      } else {
        if constexpr (MODE == kPrefill) {
          lo = row_ok ? max(lo, rb) : lo;
          hi = row_ok ? min(hi, row + 1) : hi;
        } else if constexpr (MODE == kDecode) {
          hi = row_ok ? min(hi, rb) : hi;
        } else {
          tree = row_ok ? shift_bits(rmask, base - rb) : ~0ull;
        }
      }
      const uint64_t vis = bit_range(lo - base, hi - base) & tree;
      const uint32_t w[2] = {uint32_t(vis), uint32_t(vis >> 32)};
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[bk][i] = pick_bit(s[bk][i], w[bk], 16 * (i >> 3) + (i & 7), -INFINITY);
    }

    if constexpr (kBf) {
      // ---- online softmax without a per-tile maximum: P is taken with the
      // row's current exp2 base.  A row whose base is unset takes its
      // maximum first; a row whose half-sum passes 2^16 (a score far above
      // the base, or an overflow) moves its base to its maximum, and P is
      // taken again (rare).  The base lags the true maximum by less than
      // 2^16 in P, far inside fp32 and bf16 range. ----
      if (unset) {
        if (__any(m_used == -INFINITY)) rebase(s, false);
        unset = __any(m_used == -INFINITY);
      }
      u32x4 pw[2][2];
      float ls = exp_pack(s, pw);
      // the decision is the row's own: a row is over when either of its two
      // lanes is (the same as its pair maximum passing 2^16); the common
      // path pays one compare and a scalar test of the wave's lane mask
      const uint64_t lanes_over = __ballot(ls > 65536.f);
      if (lanes_over) {
        const uint64_t rows_over = lanes_over | (lanes_over >> 32) | (lanes_over << 32);
        rebase(s, ((rows_over >> lane_id) & 1u) != 0);
        ls = exp_pack(s, pw);
      }
      l_run += ls;

      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pw[bk][c2]);
          const unsigned char* vb = vl + (32 * bk + 16 * c2) * G::kRowBytes;
#pragma unroll
          for (int md = 0; md < kDB; ++md) {
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vb + voff[md]));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vb + voff[kDB + md]));
            const s16x4 both[2] = {lo, hi};
            const bf16x8 a = __builtin_bit_cast(bf16x8, both);
            acc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[md], 0, 0, 0);
          }
        }
      sched_ld_mfma<0, 4 * kDB, 2, 8>();
    } else {
      // ---- fp32: online softmax; the exp2 base moves only when a row's
      // maximum grows by more than 2^8, so P stays <= 256 and the O rescale
      // is rare ----
      float mt = s[0][0];
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[bk][i]);
      mt = pair_max(mt);
      const bool grow = mt > m_used + tau;
      if (__any(grow)) {
        const float m_new = grow ? mt : m_used;
        const float alpha = grow ? fast_exp2((m_used - m_new) * c) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int md = 0; md < kDB; ++md)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[md][i] *= alpha;
        m_used = m_new;
      }
      const float mb = (m_used == -INFINITY) ? 0.f : m_used * c;
      float ls = 0.f;
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = fast_exp2(fmaf(s[bk][i], c, -mb));
          s[bk][i] = e;
          ls += e;
        }
      l_run += ls;

      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * bk + reg_key(i, h);
#pragma unroll
          for (int md = 0; md < kDB; ++md) {
            const float a = *reinterpret_cast<const float*>(vl + G::at(key, (32 * md + n) * 4));
            acc[md] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[bk][i], acc[md], 0, 0, 0);
          }
        }
    }
  }

  // bf16: move a row's base to its maximum so far if the row has none yet,
  // or if `sel` (this row's own choice) is set and its maximum grew; O and l
  // scale by the change.  Every other row keeps its base and its bits.
  __device__ __forceinline__ void rebase(const f32x16 (&s)[2], bool sel) {
    float mt = s[0][0];
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[bk][i]);
    mt = pair_max(mt);
    const bool grow = (sel || m_used == -INFINITY) && mt > m_used;
    const float m_new = grow ? mt : m_used;
    const float alpha = (grow && m_used != -INFINITY) ? fast_exp2((m_used - m_new) * c) : 1.f;
    l_run *= alpha;
#pragma unroll
    for (int md = 0; md < kDB; ++md)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[md][i] *= alpha;
    m_used = m_new;
    mbc = (m_used == -INFINITY) ? 0.f : m_used * c;
  }

  // bf16: P = exp2(c s - c m) as bf16 pairs, the P^T operands of the PV
  // MFMAs (pw[bk][c2]: keys 16 c2.. of 32-key block bk); returns the lane's
  // part of the row sum, taken over the rounded pairs with one
  // v_dot2_f32_bf16 each (so the normaliser sums exactly the weights the PV
  // product multiplies), in two chains.
  __device__ __forceinline__ float exp_pack(const f32x16 (&s)[2], u32x4 (&pw)[2][2]) const {
    const float mb = mbc;
    const bf16x2v ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
    float ls[2] = {0.f, 0.f};
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float e0 = fast_exp2(fmaf(s[bk][2 * j], c, -mb));
        const float e1 = fast_exp2(fmaf(s[bk][2 * j + 1], c, -mb));
        const uint32_t pk = pack_bf16x2(e0, e1);
        pw[bk][j >> 2][j & 3] = pk;
        ls[j & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, pk), ones, ls[j & 1], false);
      }
    return ls[0] + ls[1];
  }

};

// ---------------------------------------------------------------------------
// the attention kernel
// ---------------------------------------------------------------------------

// GH query heads of one KV head per workgroup; 32 / GH tokens per wave; a
// 64-token row tile therefore takes 2 * GH waves.  Two LDS stages: the tile
// after the current one streams in while the current one is consumed, with
// one barrier per tile.  Tiles are taken in four runs (segment A fully
// visible, segment A masked, segment B fully visible, segment B masked); the
// per-row visibility test runs only in the masked runs.
template <typename T, int D, int GH, int MODE>
__global__ __launch_bounds__(128 * GH, 2) void attn_kernel(AttnParams p) {
  constexpr bool kBf = std::is_same<T, __bf16>::value;
  constexpr int NW = 2 * GH;
  constexpr int TPW = 32 / GH;
  using G = TileGeom<T, D>;
  using RS = RowState<T, D, MODE>;
  constexpr int kQSteps = RS::kQSteps;
  constexpr int kDB = RS::kDB;

  __shared__ __attribute__((aligned(1024))) unsigned char lds0[G::kStageBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds1[G::kStageBytes];

  const int tid = threadIdx.x;
  // the wave index as a scalar: per-wave LDS addresses (the copies' M0) stay in
  // scalar registers
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kvh = int(blockIdx.x % unsigned(p.hkv));
  const WorkItem wi = p.work[blockIdx.x / unsigned(p.hkv)];

  const int n_a = (wi.a_hi - wi.a_lo + kKeyTile - 1) / kKeyTile;
  const int n_b = (wi.b_hi - wi.b_lo + kKeyTile - 1) / kKeyTile;
  const int n_tiles = n_a + n_b;
  // tiles [0, fa) of segment A and [n_a, n_a + fb) of segment B need no mask
  const int fa = min(n_a, max(0, wi.a_full - wi.a_lo) / kKeyTile);
  const int fb = (wi.flags & kSegBFull)  ? (wi.b_hi - wi.b_lo) / kKeyTile
                 : MODE == kDecode        ? max(0, wi.b_full - wi.b_lo) / kKeyTile
                                          : 0;
  const int64_t kv_stride = int64_t(p.hkv) * D * Elt<T>::kBytes;
  const int64_t head_off = int64_t(kvh) * D * Elt<T>::kBytes;
  const unsigned char* ka = reinterpret_cast<const unsigned char*>(p.ka) + head_off;
  const unsigned char* va = reinterpret_cast<const unsigned char*>(p.va) + head_off;
  const unsigned char* kb = reinterpret_cast<const unsigned char*>(p.kb) + head_off;
  const unsigned char* vb = reinterpret_cast<const unsigned char*>(p.vb) + head_off;

  // decode reads most K/V lines once (a page's main stream is walked once for
  // all of its branches and heads), so its copies bypass cache retention
  // unless the item marks the segment as read by other row groups too;
  // prefill and verify re-read tiles across row tiles and keep the default
  TileLoader<T, D, NW, MODE == kDecode ? kCpolStream : 0> loader;
  const int32_t shared_segs = MODE == kDecode ? wi.flags & (kSegAShared | kSegBShared) : 0;
  loader.init(lane, wave, kv_stride);
  // Tile `it` of this item: segment A's tiles, then B's.  Paged segments
  // (decode and verify only) find each tile's first cache row in the plan's
  // tile table; tiles start on 64-token boundaries of their sequence and
  // blocks hold whole tiles.
  const int a_lo = wi.a_lo, a_hi = wi.a_hi, b_lo = wi.b_lo, b_hi = wi.b_hi;
  auto issue_tile = [&](unsigned char* stage, int it) {
    const bool in_a = it < n_a;
    const int t0 = in_a ? a_lo + it * kKeyTile : b_lo + (it - n_a) * kKeyTile;
    const int t1 = in_a ? a_hi : b_hi;
    const unsigned char* kbase = in_a ? ka : kb;
    const unsigned char* vbase = in_a ? va : vb;
    int64_t row = t0;
    if constexpr (MODE != kPrefill) {
      const int32_t* tiles = in_a ? p.tile_a : p.tile_b;
      if (tiles) row = tiles[t0 / kKeyTile];
    }
    if (shared_segs & (in_a ? kSegAShared : kSegBShared))
      loader.template issue_rows<0>(stage, kbase + row * kv_stride, vbase + row * kv_stride, t1 - t0, kv_stride, wave);
    else
      loader.issue_rows(stage, kbase + row * kv_stride, vbase + row * kv_stride, t1 - t0, kv_stride, wave);
  };
  // this item's tiles: [tile_lo, tile_hi) of segment A's tiles then B's
  const int it_lo = wi.tile_lo, it_hi = min(wi.tile_hi, n_tiles);
  if (it_lo < it_hi) issue_tile(lds0, it_lo);

  RS rs;
  rs.h = lane >> 5;
  rs.n = lane & 31;
  rs.lane_id = lane;
  const int tok = wave * TPW + rs.n / GH;
  const int head = kvh * p.group + int(blockIdx.y) * GH + (rs.n % GH);
  rs.row_ok = tok < wi.nrows;
  rs.row = wi.row0 + tok;
  rs.ra = 0;
  rs.rb = 0;
  rs.rmask = 0;
  if (rs.row_ok) {
    rs.ra = p.row_a[rs.row];
    rs.rb = p.row_b[rs.row];
    if constexpr (MODE == kVerify) rs.rmask = p.row_mask[rs.row];
  }
  rs.c = p.c;
  rs.tau = 8.f / p.c;
  rs.m_used = -INFINITY;
  rs.mbc = 0.f;
  rs.unset = true;
  rs.l_run = 0.f;
  rs.init_offsets(lane);

  // Q fragment: lane half h holds dims [(D/2) h, (D/2)(h+1)) of its row.
  {
    const T* qrow = reinterpret_cast<const T*>(p.q) + (int64_t(rs.row) * p.hq + head) * D + (D / 2) * rs.h;
    if constexpr (kBf) {
#pragma unroll
      for (int s = 0; s < kQSteps; ++s) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (rs.row_ok) raw = *reinterpret_cast<const u32x4*>(qrow + 8 * s);
        rs.qf[s] = __builtin_bit_cast(bf16x8, raw);
      }
    } else {
#pragma unroll
      for (int s = 0; s < kQSteps; ++s) rs.qf[s] = rs.row_ok ? qrow[s] : 0.f;
    }
  }
#pragma unroll
  for (int md = 0; md < kDB; ++md)
#pragma unroll
    for (int i = 0; i < 16; ++i) rs.acc[md][i] = 0.f;
  const bool wave_active = wave * TPW < wi.nrows;

  // Tiles alternate between two LDS buffers, so each is a distinct object:
  // the next tile's copy into one never has to complete before reads of the
  // other.
  auto step = [&](int it, const unsigned char* cur, unsigned char* nxt) {
    // this wave's copies into `cur` are done (vmcnt(0)), then the barrier
    // publishes all of them and retires every wave's reads of `nxt`
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (it + 1 < it_hi) issue_tile(nxt, it + 1);
    if (wave_active) {
      const bool seg_a = it < n_a;
      const int t0 = seg_a ? a_lo + it * kKeyTile : b_lo + (it - n_a) * kKeyTile;
      const int t_hi = seg_a ? a_hi : b_hi;
      const bool masked = seg_a ? it >= fa : (it - n_a) >= fb;
      rs.consume(cur, cur + G::kTileBytes, t0, t_hi, seg_a, masked);
    }
  };
#pragma unroll 1
  for (int it = it_lo; it < it_hi; it += 2) {
    step(it, lds0, lds1);
    if (it + 1 < it_hi) step(it + 1, lds1, lds0);
  }

  // ---- epilogue ----
  const float l_tot = pair_sum(rs.l_run);
  if (!rs.row_ok) return;
  const int h = rs.h;
  if (MODE == kDecode || wi.out >= 0) {
    const int64_t slot = int64_t(wi.out) + tok;
    const int64_t idx = slot * p.hq + head;
    float* dst = p.part_acc + idx * D;
#pragma unroll
    for (int md = 0; md < kDB; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * md + 8 * g + 4 * h;
        float4 vv = {rs.acc[md][4 * g], rs.acc[md][4 * g + 1], rs.acc[md][4 * g + 2], rs.acc[md][4 * g + 3]};
        *reinterpret_cast<float4*>(dst + d0) = vv;
      }
    if (h == 0) {
      float2 ml = {rs.m_used == -INFINITY ? -INFINITY : rs.m_used * p.c, l_tot};
      *reinterpret_cast<float2*>(p.part_ml + idx * 2) = ml;
    }
  } else {
    const float inv = 1.f / l_tot;
    T* dst = reinterpret_cast<T*>(p.o) + (int64_t(rs.row) * p.hq + head) * D;
#pragma unroll
    for (int md = 0; md < kDB; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * md + 8 * g + 4 * h;
        if constexpr (kBf) {
          u32x2 w = {pack_bf16x2(rs.acc[md][4 * g] * inv, rs.acc[md][4 * g + 1] * inv),
                     pack_bf16x2(rs.acc[md][4 * g + 2] * inv, rs.acc[md][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(dst + d0) = w;
        } else {
          float4 vv = {rs.acc[md][4 * g] * inv, rs.acc[md][4 * g + 1] * inv, rs.acc[md][4 * g + 2] * inv,
                       rs.acc[md][4 * g + 3] * inv};
          *reinterpret_cast<float4*>(dst + d0) = vv;
        }
      }
    if (p.lse && h == 0)
      p.lse[int64_t(head) * p.n_rows + rs.row] = (rs.m_used * p.c + __log2f(l_tot)) * 0.69314718055994531f;
  }
}

// ---------------------------------------------------------------------------
// merge of fp32 partials: one (row, query head) per 64-lane group, fixed order
// ---------------------------------------------------------------------------

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int kPer = D / 64 > 0 ? D / 64 : 1;  // dims per lane
  const int lane = threadIdx.x & 63;
  const int64_t pair = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (pair >= int64_t(p.n_merge) * p.hq) return;
  const MergeRow mr = p.merge[pair / p.hq];
  const int row = mr.row, head = int(pair % p.hq);
  float mx = -INFINITY;
  for (int c = 0; c < mr.sh_count; ++c)
    mx = fmaxf(mx, p.part_ml[(int64_t(mr.sh_first + c * mr.sh_stride) * p.hq + head) * 2]);
  for (int c = 0; c < mr.sf_count; ++c)
    mx = fmaxf(mx, p.part_ml[((int64_t(mr.sf_first) + int64_t(c) * mr.sf_stride) * p.hq + head) * 2]);
  float acc[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) acc[j] = 0.f;
  float l = 0.f;
  const int n_parts = mr.sh_count + mr.sf_count;
  for (int c = 0; c < n_parts; ++c) {
    const int64_t slot = c < mr.sh_count ? int64_t(mr.sh_first) + int64_t(c) * mr.sh_stride
                                         : int64_t(mr.sf_first) + int64_t(c - mr.sh_count) * mr.sf_stride;
    const int64_t idx = slot * p.hq + head;
    const float m = p.part_ml[idx * 2];
    const float w = (m == -INFINITY) ? 0.f : fast_exp2(m - mx);
    l += w * p.part_ml[idx * 2 + 1];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int d = lane + 64 * j;
      if (d < D) acc[j] += w * p.part_acc[idx * D + d];
    }
  }
  const float inv = 1.f / l;
  T* dst = reinterpret_cast<T*>(p.o) + (int64_t(row) * p.hq + head) * D;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int d = lane + 64 * j;
    if (d < D) dst[d] = static_cast<T>(acc[j] * inv);
  }
  if (p.lse && lane == 0) p.lse[int64_t(head) * p.n_rows + row] = (mx + __log2f(l)) * 0.69314718055994531f;
}

// Explicit instantiations: every (dtype, head_dim, heads-per-workgroup, mode)
// the launchers can select.
#define TA_INSTANTIATE(T, D, GH)                                           \
  template __global__ void attn_kernel<T, D, GH, kPrefill>(AttnParams); \
  template __global__ void attn_kernel<T, D, GH, kVerify>(AttnParams);  \
  template __global__ void attn_kernel<T, D, GH, kDecode>(AttnParams);
TA_INSTANTIATE(__bf16, 32, 1)
TA_INSTANTIATE(__bf16, 32, 2)
TA_INSTANTIATE(__bf16, 64, 1)
TA_INSTANTIATE(__bf16, 64, 2)
TA_INSTANTIATE(__bf16, 128, 1)
TA_INSTANTIATE(__bf16, 128, 2)
TA_INSTANTIATE(float, 32, 1)
TA_INSTANTIATE(float, 32, 2)
TA_INSTANTIATE(float, 64, 1)
TA_INSTANTIATE(float, 64, 2)
TA_INSTANTIATE(float, 128, 1)
TA_INSTANTIATE(float, 128, 2)
#undef TA_INSTANTIATE

// ---------------------------------------------------------------------------
// file-scope scratch of the allocation-free decode entry point
// ---------------------------------------------------------------------------

// fp32 partials of tree_attn_decode_noalloc: one copy per GPU the library
// runs on, held until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: its device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[TA_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

template <typename T, int D, int GH, int MODE>
static hipError_t launch_t(const AttnParams& p, int n_work, hipStream_t st) {
  dim3 grid(unsigned(n_work) * unsigned(p.hkv), unsigned(p.group / GH));
  hipLaunchKernelGGL((attn_kernel<T, D, GH, MODE>), grid, dim3(128 * GH), 0, st, p);
  return hipGetLastError();
}

template <typename T, int MODE>
static hipError_t launch_d(const AttnParams& p, int n_work, int d, hipStream_t st) {
  const int gh = p.group == 1 ? 1 : 2;
  switch (d * 4 + gh) {
    case 32 * 4 + 1: return launch_t<T, 32, 1, MODE>(p, n_work, st);
    case 32 * 4 + 2: return launch_t<T, 32, 2, MODE>(p, n_work, st);
    case 64 * 4 + 1: return launch_t<T, 64, 1, MODE>(p, n_work, st);
    case 64 * 4 + 2: return launch_t<T, 64, 2, MODE>(p, n_work, st);
    case 128 * 4 + 1: return launch_t<T, 128, 1, MODE>(p, n_work, st);
    case 128 * 4 + 2: return launch_t<T, 128, 2, MODE>(p, n_work, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention(int mode, int dtype, const AttnParams& p, int n_work, int d, hipStream_t st) {
  if (n_work == 0) return hipSuccess;
  if (dtype == TA_DTYPE_BF16) {
    if (mode == kPrefill) return launch_d<__bf16, kPrefill>(p, n_work, d, st);
    if (mode == kVerify) return launch_d<__bf16, kVerify>(p, n_work, d, st);
    return launch_d<__bf16, kDecode>(p, n_work, d, st);
  }
  if (mode == kPrefill) return launch_d<float, kPrefill>(p, n_work, d, st);
  if (mode == kVerify) return launch_d<float, kVerify>(p, n_work, d, st);
  return launch_d<float, kDecode>(p, n_work, d, st);
}

hipError_t launch_merge(int dtype, const MergeParams& p, int d, hipStream_t st) {
  const int64_t pairs = int64_t(p.n_merge) * p.hq;
  if (pairs == 0) return hipSuccess;
  dim3 grid(unsigned((pairs + 3) / 4));
  if (dtype == TA_DTYPE_BF16) {
    if (d == 32) hipLaunchKernelGGL((merge_kernel<__bf16, 32>), grid, dim3(256), 0, st, p);
    else if (d == 64) hipLaunchKernelGGL((merge_kernel<__bf16, 64>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((merge_kernel<__bf16, 128>), grid, dim3(256), 0, st, p);
  } else {
    if (d == 32) hipLaunchKernelGGL((merge_kernel<float, 32>), grid, dim3(256), 0, st, p);
    else if (d == 64) hipLaunchKernelGGL((merge_kernel<float, 64>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((merge_kernel<float, 128>), grid, dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace ta
