// HIP kernels for the backward of packed tree-varlen attention (gfx950).
//
// The gradients of o = softmax(scale q k^T, masked) v for an output
// gradient dO follow from the definition (PaDoc summary, "Training
// paradigm": the model trains through exactly this masked forward):
//   P = exp(scale q k^T - lse)   (lse saved by the forward)
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - Dd),  Dd = rowsum(dO * O)
//   dQ = scale dS K,  dK = scale dS^T Q
// Launches:
//   bwd_prep_kernel   Dd and lse * log2(e) per (query head, row), fp32
//   bwd_dq_kernel     query-major, over the forward's row tiles: recomputes
//                     S^T = K Q^T and dP^T = V dO^T per 64-key tile and adds
//                     K^T dS^T into dQ^T held in registers
//   bwd_dkdv_kernel   key-major, over the plan's key tiles: each wave holds
//                     16 keys of one KV head and walks the 64-row tiles (and
//                     every query head of the group) that can see them,
//                     adding dO^T P into dV^T and Q^T dS into dK^T; a long
//                     walk comes as pieces that write fp32 partials
//   bwd_kmerge_kernel the partials of each split key tile summed in order
// With query heads in pairs (hq / hkv even) the two passes go out as one
// launch, bwd_fused_kernel: the row tiles first, then the key-major items, so
// one pass's long items and the other's short ones share the GPU instead of
// each launch ending on a tail of its own.
// Both main kernels pair an operand read from an LDS tile against one held
// in registers, and a transposing LDS read (ds_read_b64_tr_b16) against a
// product taken straight from accumulators: 32x32x16 bf16 MFMAs in the
// query-major kernel (the forward's formulation), 16x16x32 in the key-major
// one (half the registers per wave, so two waves share a SIMD).  No atomics: each
// output element is written by exactly one wave, so results are
// deterministic.
#include "ta_device.h"

namespace ta {

// One (row, query head) per 64-lane group: Dd = sum_d dO * O and the
// forward's lse converted to log2 units.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
  constexpr int kPer = D / 64 > 0 ? D / 64 : 1;
  const int lane = threadIdx.x & 63;
  const int64_t pair = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (pair >= p.n_rows * p.hq) return;
  const int64_t row = pair / p.hq;
  const int head = int(pair % p.hq);
  const __bf16* o = reinterpret_cast<const __bf16*>(p.o) + (row * p.hq + head) * D;
  const __bf16* g = reinterpret_cast<const __bf16*>(p.dO) + (row * p.hq + head) * D;
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int d = lane + 64 * j;
    if (d < D) s += float(o[d]) * float(g[d]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) {
    const int64_t idx = int64_t(head) * p.n_rows + row;
    p.dd[idx] = s;
    p.l2[idx] = p.lse[idx] * 1.4426950408889634f;
  }
}

// ---------------------------------------------------------------------------
// dQ: query-major
// ---------------------------------------------------------------------------

// GH query heads of one KV head per workgroup (heads GH hy .. of the
// group), 32 / GH tokens per wave, a 64-token row tile per work item (the
// forward's tiling and segments); two LDS stages of TileGeom<bf16, D>.
template <int D, int GH>
__device__ __forceinline__ void bwd_dq_body(const BwdParams& p, unsigned char* lds0, unsigned char* lds1, int kvh,
                                            int item, int hy) {
  using T = __bf16;
  using G = TileGeom<T, D>;
  constexpr int NW = 2 * GH;
  constexpr int TPW = 32 / GH;
  constexpr int kQSteps = D / 16;
  constexpr int kDB = D / 32;

  const int tid = threadIdx.x;
  // the wave index as a scalar: per-wave LDS addresses (the copies' M0) stay in
  // scalar registers
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const WorkItem wi = p.work[item];
  const int n_a = (wi.a_hi - wi.a_lo + kKeyTile - 1) / kKeyTile;
  const int n_tiles = n_a + (wi.b_hi - wi.b_lo + kKeyTile - 1) / kKeyTile;
  const int fa = min(n_a, max(0, wi.a_full - wi.a_lo) / kKeyTile);
  const int64_t kv_stride = int64_t(p.hkv) * D * 2;
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k) + int64_t(kvh) * D * 2;
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.v) + int64_t(kvh) * D * 2;

  TileLoader<T, D, NW> loader;
  loader.init(lane, wave, kv_stride);
  auto tile0 = [&](int it) { return it < n_a ? wi.a_lo + it * kKeyTile : wi.b_lo + (it - n_a) * kKeyTile; };
  auto tile_hi = [&](int it) { return it < n_a ? wi.a_hi : wi.b_hi; };
  if (n_tiles > 0) loader.issue(lds0, kbase, vbase, tile0(0), tile_hi(0), kv_stride, wave);

  const int h = lane >> 5, n = lane & 31;
  const int tok = wave * TPW + n / GH;
  const int head = kvh * p.group + hy * GH + (n % GH);
  const bool row_ok = tok < wi.nrows;
  const int row = wi.row0 + tok;
  int ra = 0, rb = 0;
  float l2 = 0.f, dd = 0.f;
  bf16x8 qf[kQSteps], df[kQSteps];
  {
    const T* qrow = reinterpret_cast<const T*>(p.q) + (int64_t(row) * p.hq + head) * D + (D / 2) * h;
    const T* grow = reinterpret_cast<const T*>(p.dO) + (int64_t(row) * p.hq + head) * D + (D / 2) * h;
#pragma unroll
    for (int s = 0; s < kQSteps; ++s) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (row_ok) {
        a = *reinterpret_cast<const u32x4*>(qrow + 8 * s);
        b = *reinterpret_cast<const u32x4*>(grow + 8 * s);
      }
      qf[s] = __builtin_bit_cast(bf16x8, a);
      df[s] = __builtin_bit_cast(bf16x8, b);
    }
    if (row_ok) {
      ra = p.row_a[row];
      rb = p.row_b[row];
      l2 = p.l2[int64_t(head) * p.n_rows + row];
      dd = p.dd[int64_t(head) * p.n_rows + row];
    }
  }
  // LDS operand offsets (as in the forward): K / V rows in permuted MFMA
  // row order for S^T and dP^T; transposing reads of K for dQ^T
  const int krow0 = key_perm(n);
  const int kx = G::at(krow0, D * h);
  int voff[2 * kDB];
  {
    const int m16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int md = 0; md < kDB; ++md)
        voff[r * kDB + md] = G::at(8 * (grp >> 1) + 4 * r + (m16 >> 2), 2 * (32 * md + 16 * (grp & 1) + 4 * (m16 & 3)));
  }
  f32x16 acc[kDB];
#pragma unroll
  for (int md = 0; md < kDB; ++md)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[md][i] = 0.f;
  const bool wave_active = wave * TPW < wi.nrows;

  auto consume = [&](const unsigned char* kl, const unsigned char* vl, int it) {
    const bool seg_a = it < n_a;
    const int t0 = tile0(it), t_hi = tile_hi(it);
    const bool masked = seg_a ? it >= fa : true;
    // masked tiles: the row's visible keys [lo, hi) of this tile as a mask
    // over the lane's key offsets (as in the forward)
    uint32_t w[2] = {~0u, ~0u};
    if (masked) {
      const int base = t0 + 8 * h;
      const int lo = seg_a ? base : max(base, rb);
      const int hi = seg_a ? min(t_hi, ra) : min(t_hi, row + 1);
      const uint64_t vis = bit_range(lo - base, hi - base);
      w[0] = uint32_t(vis);
      w[1] = uint32_t(vis >> 32);
    }
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int st = 0; st < kQSteps; ++st) {
        const int off = (kx ^ (16 * st)) + 32 * bk * G::kRowBytes;
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kl + off), qf[st], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(vl + off), df[st], dp, 0, 0, 0);
      }
      sched_ld_mfma<0, 2 * kQSteps, 1, 4>();
      // invisible pairs: s -> -inf (P = 0) and dP -> Dd, so dS is exactly 0
      // whatever the key's values
      if (masked) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = 16 * (i >> 3) + (i & 7);
          s[i] = pick_bit(s[i], w[bk], c, -INFINITY);
          dp[i] = pick_bit(dp[i], w[bk], c, dd);
        }
      }
      // dS^T = P^T (dP^T - Dd), P^T = 2^(s c - lse2)
      u32x4 pk[2];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float ds[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int i = 2 * j + e;
          ds[e] = fast_exp2(fmaf(s[i], p.c, -l2)) * (dp[i] - dd);
        }
        pk[j >> 2][j & 3] = pack_bf16x2(ds[0], ds[1]);
      }
      // dQ^T += K^T dS^T over the 32 keys of this block
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pk[c2]);
        const unsigned char* kb = kl + (32 * bk + 16 * c2) * G::kRowBytes;
#pragma unroll
        for (int md = 0; md < kDB; ++md) {
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(kb + voff[md]));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(kb + voff[kDB + md]));
          const s16x4 both[2] = {lo, hi};
          acc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pb, acc[md], 0, 0, 0);
        }
      }
      sched_ld_mfma<0, 2 * kDB, 2, 4>();
    }
  };
  auto step = [&](int it, const unsigned char* cur, unsigned char* nxt) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's copies into cur are done
    __syncthreads();                     // ... and every wave's; reads of nxt are retired
    if (it + 1 < n_tiles) loader.issue(nxt, kbase, vbase, tile0(it + 1), tile_hi(it + 1), kv_stride, wave);
    if (wave_active) consume(cur, cur + G::kTileBytes, it);
  };
#pragma unroll 1
  for (int it = 0; it < n_tiles; it += 2) {
    step(it, lds0, lds1);
    if (it + 1 < n_tiles) step(it + 1, lds1, lds0);
  }

  if (!row_ok) return;
  T* dst = reinterpret_cast<T*>(p.dq) + (int64_t(row) * p.hq + head) * D;
#pragma unroll
  for (int md = 0; md < kDB; ++md)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * md + 8 * g + 4 * h;
      u32x2 w = {pack_bf16x2(acc[md][4 * g] * p.scale, acc[md][4 * g + 1] * p.scale),
                 pack_bf16x2(acc[md][4 * g + 2] * p.scale, acc[md][4 * g + 3] * p.scale)};
      *reinterpret_cast<u32x2*>(dst + d0) = w;
    }
}

// ---------------------------------------------------------------------------
// dK, dV: key-major
// ---------------------------------------------------------------------------

// Per-row values of a 64-row tile staged beside its Q and dO tiles (four
// 256-byte arrays, one DMA each).
struct RowMeta {
  float l2[64], dd[64];
  int32_t ra[64], rb[64];
};

// Four waves of 16 keys (one 64-key tile of one KV head) per workgroup, two
// waves per SIMD.  Per wave, with 16x16x32 MFMAs (A: lane l holds row l % 16,
// k in [8 (l / 16), +8); B: column l % 16, same k; D: column l % 16, rows
// 4 (l / 16) .. +3):
//   S = Q K^T and dP = dO V^T per 16-row block (Q, dO rows from LDS; K, V
//     of the wave's keys in registers): lane l holds key l % 16 and rows
//     4 (l / 16) + i of the block;
//   dV^T += dO^T P and dK^T += Q^T dS per 32 rows: the A operand is a pair
//     of transposing LDS reads (rows 4 (l / 16) .. +3 of each 16-row block at
//     16 consecutive d), the B operand the lane's own P / dS values of those
//     two blocks, packed in the same row order.
// Two LDS stages of DkdvStage<D>::kBytes: a TileGeomB<bf16, D> Q / dO tile
// pair and the tile's RowMeta.
template <int D>
struct DkdvStage {
  static constexpr int kBytes = TileGeomB<__bf16, D>::kStageBytes + int(sizeof(RowMeta));
};
template <int D>
__device__ __forceinline__ void bwd_dkdv_body(const BwdParams& p, unsigned char* lds0, unsigned char* lds1, int kvh,
                                              int item) {
  using T = __bf16;
  using G = TileGeomB<T, D>;
  constexpr int NW = 4;
  constexpr int kKS = D / 32;  // k-steps of 32 over head_dim
  constexpr int kDB = D / 16;  // 16-wide blocks of head_dim

  const int tid = threadIdx.x;
  // the wave index as a scalar: per-wave LDS addresses (the copies' M0) stay in
  // scalar registers
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const WorkItem wi = p.kwork[item];
  const bool branch_keys = (wi.flags & kKeyBranch) != 0;
  const int n_a = (wi.a_hi - wi.a_lo + kKeyTile - 1) / kKeyTile;
  const int n_pc = wi.tile_hi - wi.tile_lo;  // this piece's row tiles per query head
  const int n_steps = n_pc * p.group;        // (head, row tile) pairs
  const int64_t q_stride = int64_t(p.hq) * D * 2;
  auto rt0 = [&](int r) { return r < n_a ? wi.a_lo + r * kKeyTile : wi.b_lo + (r - n_a) * kKeyTile; };
  auto rt_hi = [&](int r) { return r < n_a ? wi.a_hi : wi.b_hi; };

  TileLoader<T, D, NW, 0, G> loader;
  loader.init(lane, wave, q_stride);
  // step = (query head j of the group, row tile r of the piece), heads
  // outer: the Q and dO tiles and the tile's row values go to the stage by
  // DMA; wave w copies row-value array w of RowMeta (lse2, Dd, row_a, row_b),
  // and rows past the segment end read as 0
  auto issue = [&](int j, int r, unsigned char* stage) {
    const int head = kvh * p.group + j;
    const unsigned char* qb = reinterpret_cast<const unsigned char*>(p.q) + int64_t(head) * D * 2;
    const unsigned char* gb = reinterpret_cast<const unsigned char*>(p.dO) + int64_t(head) * D * 2;
    const int r0 = rt0(r), rhi = rt_hi(r);
    loader.issue(stage, qb, gb, r0, rhi, q_stride, wave);
    const int64_t hb = int64_t(head) * p.n_rows;
    const void* src = wave == 0   ? static_cast<const void*>(p.l2 + hb + r0)
                      : wave == 1 ? static_cast<const void*>(p.dd + hb + r0)
                      : wave == 2 ? static_cast<const void*>(p.row_a + r0)
                                  : static_cast<const void*>(p.row_b + r0);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src), (short)0, 4 * min(rhi - r0, kKeyTile), 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(stage + G::kStageBytes + 4 * kKeyTile * wave), 4,
                                             4 * lane, 0, 0, 0);
  };

  // this wave's 16 keys as B operands (lane: key l % 16, dims 32 ks + 8 g ..)
  const int g = lane >> 4, n16 = lane & 15;
  const int key = wi.row0 + 16 * wave + n16;
  const bool key_ok = 16 * wave + n16 < wi.nrows;
  bf16x8 kf[kKS], vf[kKS];
  {
    const T* krow = reinterpret_cast<const T*>(p.k) + (int64_t(key) * p.hkv + kvh) * D + 8 * g;
    const T* vrow = reinterpret_cast<const T*>(p.v) + (int64_t(key) * p.hkv + kvh) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (key_ok) {
        a = *reinterpret_cast<const u32x4*>(krow + 32 * ks);
        b = *reinterpret_cast<const u32x4*>(vrow + 32 * ks);
      }
      kf[ks] = __builtin_bit_cast(bf16x8, a);
      vf[ks] = __builtin_bit_cast(bf16x8, b);
    }
  }
  // LDS offsets.  Q / dO row n16 of a 16-row block at dims 32 ks + 8 g: the
  // k-steps differ only in swizzled chunk bits (qx ^ 64 ks), the blocks by
  // whole 16-row steps.  Transposing reads: lane m of a 16-lane group
  // addresses row 4 g + m / 4 at dims 16 db + 4 (m % 4); the d-blocks differ
  // in chunk bits (tx ^ 32 db).
  const int qx = G::at(n16, 16 * g);
  const int tx = G::at(4 * g + (n16 >> 2), 8 * (n16 & 3));
  f32x4 dk[kDB], dv[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dk[db][i] = 0.f;
      dv[db][i] = 0.f;
    }

  auto consume = [&](const unsigned char* stage, int r) {
    const unsigned char* qt = stage;
    const unsigned char* gt = stage + G::kTileBytes;
    const RowMeta* m = reinterpret_cast<const RowMeta*>(stage + G::kStageBytes);
    const int r0 = rt0(r), rhi = rt_hi(r);
    // row tiles past the segment's first fully visible row need no test
    // (rows past the segment end hold zero Q, dO, lse2 and Dd: they add 0)
    const bool masked = r0 < (r < n_a ? wi.a_full : wi.out);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      u32x4 pp, pd;
#pragma unroll
      for (int b1 = 0; b1 < 2; ++b1) {
        const int rb = 2 * h2 + b1;
        f32x4 sc = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
          const int off = (qx ^ (64 * ks)) + 16 * rb * G::kRowBytes;
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(qt + off), kf[ks], sc, 0, 0,
                                                        0);
          dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(gt + off), vf[ks], dp, 0, 0,
                                                        0);
        }
        // the lane's rows 16 rb + 4 g + i: one float4 / int4 of each row value
        const int lr = 16 * rb + 4 * g;
        const float4 l2 = *reinterpret_cast<const float4*>(&m->l2[lr]);
        const float4 dd = *reinterpret_cast<const float4*>(&m->dd[lr]);
        const float l2v[4] = {l2.x, l2.y, l2.z, l2.w}, ddv[4] = {dd.x, dd.y, dd.z, dd.w};
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = fmaf(sc[i], p.c, -l2v[i]);
        if (masked) {
          // the row sees this lane's key when key is in [lo, hi): [row_b, row]
          // for branch keys, below row_a for main keys; an invisible pair
          // gets P = 0 and dP = Dd, so it adds exactly 0
          const int4 ra4 = *reinterpret_cast<const int4*>(&m->ra[lr]);
          const int4 rb4 = *reinterpret_cast<const int4*>(&m->rb[lr]);
          const int ra[4] = {ra4.x, ra4.y, ra4.z, ra4.w}, rbv[4] = {rb4.x, rb4.y, rb4.z, rb4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = r0 + lr + i;
            const int lo = branch_keys ? rbv[i] : INT32_MIN;
            const int hi = branch_keys ? row + 1 : ra[i];
            const bool vis = (row < rhi) & (key >= lo) & (key < hi);
            x[i] = vis ? x[i] : -INFINITY;
            dp[i] = vis ? dp[i] : ddv[i];
          }
        }
        float pr[4], ds[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[i] = fast_exp2(x[i]);
          ds[i] = pr[i] * (dp[i] - ddv[i]);
        }
        pp[2 * b1] = pack_bf16x2(pr[0], pr[1]);
        pp[2 * b1 + 1] = pack_bf16x2(pr[2], pr[3]);
        pd[2 * b1] = pack_bf16x2(ds[0], ds[1]);
        pd[2 * b1 + 1] = pack_bf16x2(ds[2], ds[3]);
      }
      sched_ld_mfma<0, 4 * kKS, 1, 8>();
      // dV^T += dO^T P and dK^T += Q^T dS over these 32 rows
      const bf16x8 bp = __builtin_bit_cast(bf16x8, pp);
      const bf16x8 bd = __builtin_bit_cast(bf16x8, pd);
      const int rowb = 32 * h2 * G::kRowBytes;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const int o0 = (tx ^ (32 * db)) + rowb;
        const int o1 = o0 + 16 * G::kRowBytes;
        const s16x4 g0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(gt + o0));
        const s16x4 g1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(gt + o1));
        const s16x4 gg[2] = {g0, g1};
        dv[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, gg), bp, dv[db], 0, 0, 0);
        const s16x4 q0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(qt + o0));
        const s16x4 q1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(qt + o1));
        const s16x4 qq[2] = {q0, q1};
        dk[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qq), bd, dk[db], 0, 0, 0);
      }
      sched_ld_mfma<0, 2 * kDB, 2, 16>();
    }
  };

  // (head, row tile) of the next step to copy and of the step consumed,
  // advanced by counting rather than by a division per step
  int j_in = 0, r_in = wi.tile_lo, r_cur = wi.tile_lo;
  auto advance_in = [&]() {
    if (++r_in == wi.tile_hi) {
      r_in = wi.tile_lo;
      ++j_in;
    }
  };
  if (n_steps > 0) {
    issue(j_in, r_in, lds0);
    advance_in();
  }
  auto step = [&](int s, unsigned char* cur, unsigned char* nxt) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's copies into cur are done
    __syncthreads();                     // ... and every wave's; reads of nxt are retired
    if (s + 1 < n_steps) {
      issue(j_in, r_in, nxt);
      advance_in();
    }
    consume(cur, r_cur);
    if (++r_cur == wi.tile_hi) r_cur = wi.tile_lo;
  };
#pragma unroll 1
  for (int s = 0; s < n_steps; s += 2) {
    step(s, lds0, lds1);
    if (s + 1 < n_steps) step(s + 1, lds1, lds0);
  }

  if (!key_ok) return;
  if (wi.b_full >= 0) {
    // a piece of a split key tile: fp32 partials, summed by bwd_kmerge_kernel
    float* kp = p.kpart + (int64_t(wi.b_full) * p.hkv + kvh) * 2 * kKeyTile * D + (16 * wave + n16) * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      *reinterpret_cast<f32x4*>(kp + 16 * db + 4 * g) = dk[db];
      *reinterpret_cast<f32x4*>(kp + kKeyTile * D + 16 * db + 4 * g) = dv[db];
    }
    return;
  }
  T* kd = reinterpret_cast<T*>(p.dk) + (int64_t(key) * p.hkv + kvh) * D;
  T* vd = reinterpret_cast<T*>(p.dv) + (int64_t(key) * p.hkv + kvh) * D;
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
    const int d0 = 16 * db + 4 * g;
    u32x2 a = {pack_bf16x2(dk[db][0] * p.scale, dk[db][1] * p.scale),
               pack_bf16x2(dk[db][2] * p.scale, dk[db][3] * p.scale)};
    u32x2 b = {pack_bf16x2(dv[db][0], dv[db][1]), pack_bf16x2(dv[db][2], dv[db][3])};
    *reinterpret_cast<u32x2*>(kd + d0) = a;
    *reinterpret_cast<u32x2*>(vd + d0) = b;
  }
}

// Split key tiles: dK, dV of keys [key0, key0 + nkeys) of one KV head per
// workgroup, the sum of the pieces' fp32 partials in slot order (fixed, so
// results are deterministic).
template <int D>
__global__ __launch_bounds__(256) void bwd_kmerge_kernel(BwdParams p) {
  const int kvh = int(blockIdx.x % unsigned(p.hkv));
  const KMerge km = p.kmerge[blockIdx.x / unsigned(p.hkv)];
  const int n4 = km.nkeys * D / 4;
  for (int e4 = threadIdx.x; e4 < n4; e4 += 256) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    for (int c = 0; c < km.count; ++c) {
      const float4* src =
          reinterpret_cast<const float4*>(p.kpart + (int64_t(km.first + c) * p.hkv + kvh) * 2 * kKeyTile * D);
      const float4 x = src[e4], y = src[kKeyTile * D / 4 + e4];
      a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
      b.x += y.x; b.y += y.y; b.z += y.z; b.w += y.w;
    }
    const int key = km.key0 + (4 * e4) / D, d = (4 * e4) % D;
    const int64_t at = (int64_t(key) * p.hkv + kvh) * D + d;
    *reinterpret_cast<u32x2*>(reinterpret_cast<__bf16*>(p.dk) + at) =
        u32x2{pack_bf16x2(a.x * p.scale, a.y * p.scale), pack_bf16x2(a.z * p.scale, a.w * p.scale)};
    *reinterpret_cast<u32x2*>(reinterpret_cast<__bf16*>(p.dv) + at) =
        u32x2{pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w)};
  }
}

// The query-major pass alone (one query head per KV head: two-wave groups).
template <int D, int GH>
__global__ __launch_bounds__(128 * GH, 2) void bwd_dq_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * TileGeom<__bf16, D>::kStageBytes];
  bwd_dq_body<D, GH>(p, lds, lds + TileGeom<__bf16, D>::kStageBytes, int(blockIdx.x % unsigned(p.hkv)),
                     int(blockIdx.x / unsigned(p.hkv)), int(blockIdx.y));
}

// The key-major pass alone.
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * DkdvStage<D>::kBytes];
  bwd_dkdv_body<D>(p, lds, lds + DkdvStage<D>::kBytes, int(blockIdx.x % unsigned(p.hkv)),
                   int(blockIdx.x / unsigned(p.hkv)));
}

// Both passes in one launch (query heads in pairs): workgroups [0, n_dq)
// take the query-major row tiles (heads pair by pair), the rest the key-major
// items.  The row tiles come first, longest first, so the key-major items
// fill the slots their tail leaves and the launch ends on short pieces.
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_fused_kernel(BwdParams p, int n_dq) {
  constexpr int kA = TileGeom<__bf16, D>::kStageBytes, kB = DkdvStage<D>::kBytes;
  constexpr int kStage = kA > kB ? kA : kB;
  static_assert(kStage % 1024 == 0, "stages start on 1 KB boundaries");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * kStage];
  const int b = int(blockIdx.x), kvh = b % p.hkv;
  if (b < n_dq) {
    const int t = b / p.hkv, ny = p.group / 2;
    bwd_dq_body<D, 2>(p, lds, lds + kStage, kvh, t / ny, t % ny);
  } else {
    bwd_dkdv_body<D>(p, lds, lds + kStage, kvh, (b - n_dq) / p.hkv);
  }
}

template __global__ void bwd_prep_kernel<32>(BwdParams);
template __global__ void bwd_prep_kernel<64>(BwdParams);
template __global__ void bwd_prep_kernel<128>(BwdParams);
#define TA_INSTANTIATE_BWD(D)                              \
  template __global__ void bwd_dq_kernel<D, 1>(BwdParams); \
  template __global__ void bwd_dkdv_kernel<D>(BwdParams);   \
  template __global__ void bwd_fused_kernel<D>(BwdParams, int); \
  template __global__ void bwd_kmerge_kernel<D>(BwdParams);
TA_INSTANTIATE_BWD(32)
TA_INSTANTIATE_BWD(64)
TA_INSTANTIATE_BWD(128)
#undef TA_INSTANTIATE_BWD

template <int D>
static hipError_t launch_bwd_d(const BwdParams& p, int n_work, int n_kwork, int n_kmerge, hipStream_t st) {
  const int64_t pairs = p.n_rows * p.hq;
  if (pairs > 0) hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3(unsigned((pairs + 3) / 4)), dim3(256), 0, st, p);
  if (p.group == 1) {
    if (n_work > 0)
      hipLaunchKernelGGL((bwd_dq_kernel<D, 1>), dim3(unsigned(n_work) * unsigned(p.hkv)), dim3(128), 0, st, p);
    if (n_kwork > 0)
      hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3(unsigned(n_kwork) * unsigned(p.hkv)), dim3(256), 0, st, p);
  } else if (n_work + n_kwork > 0) {
    const int64_t n_dq = int64_t(n_work) * p.hkv * (p.group / 2);
    const int64_t n_blocks = n_dq + int64_t(n_kwork) * p.hkv;
    hipLaunchKernelGGL((bwd_fused_kernel<D>), dim3(unsigned(n_blocks)), dim3(256), 0, st, p, int(n_dq));
  }
  if (n_kmerge > 0)
    hipLaunchKernelGGL((bwd_kmerge_kernel<D>), dim3(unsigned(n_kmerge) * unsigned(p.hkv)), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_backward(const BwdParams& p, int n_work, int n_kwork, int n_kmerge, int d, hipStream_t st) {
  if (d == 32) return launch_bwd_d<32>(p, n_work, n_kwork, n_kmerge, st);
  if (d == 64) return launch_bwd_d<64>(p, n_work, n_kwork, n_kmerge, st);
  if (d == 128) return launch_bwd_d<128>(p, n_work, n_kwork, n_kmerge, st);
  return hipErrorInvalidValue;
}

}  // namespace ta
