// Kernel launch interface between the C ABI layer and attn_kernels.hip.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "ta_internal.h"

namespace ta {

enum Mode : int { kPrefill = 0, kVerify = 1, kDecode = 2 };

struct AttnParams {
  const void* q;
  const void* ka;
  const void* va;
  const void* kb;
  const void* vb;
  void* o;
  float* lse;
  float* part_acc;  // decode: [n_partials, hq, d] unnormalised fp32 accumulators
  float* part_ml;   // decode: [n_partials, hq, 2] (running max in log2 units of the scaled score, sum)
  const WorkItem* work;
  const int32_t* row_a;
  const int32_t* row_b;
  const uint64_t* row_mask;
  // paged plans: cache row of the first token of each 64-token tile of
  // segment A / B, by virtual position / 64; NULL for a contiguous segment
  const int32_t* tile_a;
  const int32_t* tile_b;
  int32_t hq, hkv, group;
  float c;  // softmax scale * log2(e)
  int64_t n_rows;
};

struct MergeParams {
  const MergeRow* merge;  // n_merge entries
  const float* part_acc;
  const float* part_ml;
  void* o;
  float* lse;
  int32_t n_rows;   // rows of o / lse (lse is [hq, n_rows])
  int32_t n_merge;  // merge-table entries
  int32_t hq;
};

// Backward of the packed prefill (bf16): gradients dq [rows, hq, d], dk and
// dv [rows, hkv, d] from q, k, v, o, lse and dO.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  void* dq;
  void* dk;
  void* dv;
  const float* lse;  // [hq, rows] natural log, as the forward writes it
  float* l2;         // scratch [hq, rows]: lse * log2(e)
  float* dd;         // scratch [hq, rows]: sum_d dO * O
  const WorkItem* work;   // row-major items (the forward's)
  const WorkItem* kwork;  // key-major items
  const KMerge* kmerge;   // split key tiles
  float* kpart;           // scratch [slots, hkv, 2 (dK, dV), 64 keys, d] fp32 partials
  const int32_t* row_a;
  const int32_t* row_b;
  int32_t hq, hkv, group;
  float c;      // scale * log2(e)
  float scale;
  int64_t n_rows;
};

// Greedy acceptance of verified draft trees (tree_attn_accept).
struct AcceptParams {
  const void* logits;       // [n_nodes + n_trees rows, ld] bf16 or fp32
  int64_t ld, vocab;        // row stride and scored entries per row (elements)
  const int32_t* tree_tab;  // node offsets [n_trees + 1], then parents
  const int32_t* tokens;    // [n_nodes] drafted token of each node
  int32_t n_trees;
  int32_t exact;            // 1: accept only the row's top token
  int32_t chunks;           // argmax pieces per row
  int64_t chunk_elems;      // elements per piece (multiple of 8)
  float* part_max;          // scratch [rows, chunks]
  int32_t* part_idx;        // scratch [rows, chunks]
  double log_tau;
  int32_t* path;            // [n_nodes]: accepted node indices, tree-major
  int32_t* n_path;          // [n_trees]
  int32_t* next_token;      // [n_trees]
};

hipError_t launch_attention(int mode, int dtype, const AttnParams& p, int n_work, int head_dim, hipStream_t st);
hipError_t launch_merge(int dtype, const MergeParams& p, int head_dim, hipStream_t st);
hipError_t launch_backward(const BwdParams& p, int n_work, int n_kwork, int n_kmerge, int head_dim, hipStream_t st);
hipError_t launch_accept(int dtype, const AcceptParams& p, int64_t n_rows, hipStream_t st);
// Device address of the file-scope scratch (TA_STATIC_SCRATCH_BYTES) on the
// current device, looked up on the first call per device.
hipError_t static_scratch(void** ptr);
hipError_t launch_calib_mfma(int32_t blocks, int32_t iters, uint32_t seed, float* sink, hipStream_t st);
hipError_t launch_calib_read(const void* src, int64_t bytes, int32_t blocks, uint32_t* sink, hipStream_t st);
int64_t calib_mfma_flops(int32_t blocks, int32_t iters);
hipError_t launch_calib_tile(int32_t variant, int32_t blocks, int32_t iters, uint32_t seed, const void* src,
                             int64_t src_bytes, float* sink, hipStream_t st);
int64_t calib_tile_flops(int32_t blocks, int32_t iters);
int64_t calib_tile_min_bytes();

}  // namespace ta
