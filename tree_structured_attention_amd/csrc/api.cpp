// C ABI of libtree_attn: argument validation, plan accessors and launches.
// Every check runs on the host before anything is enqueued, so an invalid
// call leaves outputs and the stream untouched.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <stdexcept>
#include <string>

#include "ta_kernels.h"

namespace ta {

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_heads(int32_t dtype, int32_t hq, int32_t hkv, int32_t d, float scale) {
  if (dtype != TA_DTYPE_BF16 && dtype != TA_DTYPE_F32) return fail(TA_ERR_UNSUPPORTED, "dtype must be TA_DTYPE_BF16 or TA_DTYPE_F32");
  if (hq <= 0 || hkv <= 0) return fail(TA_ERR_INVALID_ARG, "hq and hkv must be positive");
  if (hq % hkv != 0) return fail(TA_ERR_INVALID_ARG, "hq must be a multiple of hkv");
  const int g = hq / hkv;
  if (32 % g != 0) return fail(TA_ERR_UNSUPPORTED, "hq / hkv must divide 32");
  if (d != 32 && d != 64 && d != 128) return fail(TA_ERR_UNSUPPORTED, "head_dim must be 32, 64 or 128");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(TA_ERR_INVALID_ARG, "scale must be positive and finite");
  return TA_OK;
}

int check_tensor(const void* ptr, int64_t count, const char* name) {
  if (count == 0) return TA_OK;
  if (!ptr) return fail(TA_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned(ptr, 16)) return fail(TA_ERR_INVALID_ARG, std::string(name) + " must be 16-byte aligned");
  return TA_OK;
}

int check_plan(const ta_plan* plan, int kind, const char* who) {
  if (!plan) return fail(TA_ERR_INVALID_ARG, std::string(who) + ": plan is NULL");
  if (plan->kind != kind) return fail(TA_ERR_STATE, std::string(who) + ": plan was built for another entry point");
  return TA_OK;
}

int check_uploaded(const ta_plan* plan, const char* who) {
  if (!plan->dev) return fail(TA_ERR_STATE, std::string(who) + ": plan is not uploaded (tree_attn_plan_upload)");
  return TA_OK;
}

AttnParams base_params(const ta_plan* plan, int32_t hq, int32_t hkv, float scale) {
  AttnParams p{};
  const unsigned char* dev = static_cast<const unsigned char*>(plan->dev);
  p.work = reinterpret_cast<const WorkItem*>(dev + plan->layout.work);
  p.row_a = reinterpret_cast<const int32_t*>(dev + plan->layout.row_a);
  p.row_b = reinterpret_cast<const int32_t*>(dev + plan->layout.row_b);
  p.row_mask = reinterpret_cast<const uint64_t*>(dev + plan->layout.mask);
  p.tile_a = plan->tile_a.empty() ? nullptr : reinterpret_cast<const int32_t*>(dev + plan->layout.tile_a);
  p.tile_b = plan->tile_b.empty() ? nullptr : reinterpret_cast<const int32_t*>(dev + plan->layout.tile_b);
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  p.c = scale * 1.4426950408889634f;
  p.n_rows = plan->n_rows;
  return p;
}

int hip_status(hipError_t e, const char* who) {
  if (e == hipSuccess) return TA_OK;
  return fail(TA_ERR_HIP, std::string(who) + ": " + hipGetErrorString(e));
}

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

int64_t scratch_need(const ta_plan* plan, int32_t hq, int32_t d) {
  const int64_t slots = plan->n_partials * hq;
  if (slots == 0) return 0;
  return align256(slots * d * 4) + align256(slots * 2 * 4);
}

int check_scratch(const ta_plan* plan, int32_t hq, int32_t d, void* scratch, size_t bytes, const char* who) {
  const int64_t need = scratch_need(plan, hq, d);
  if (need == 0) return TA_OK;
  if (!scratch) return fail(TA_ERR_WORKSPACE, std::string(who) + ": scratch is NULL (tree_attn_scratch_bytes > 0)");
  if (!aligned(scratch, 256)) return fail(TA_ERR_INVALID_ARG, std::string(who) + ": scratch must be 256-byte aligned");
  if (int64_t(bytes) < need) return fail(TA_ERR_WORKSPACE, std::string(who) + ": scratch smaller than tree_attn_scratch_bytes");
  return TA_OK;
}

void set_partials(AttnParams& p, const ta_plan* plan, int32_t hq, int32_t d, void* scratch) {
  const int64_t slots = plan->n_partials * hq;
  p.part_acc = static_cast<float*>(scratch);
  p.part_ml = slots ? reinterpret_cast<float*>(static_cast<unsigned char*>(scratch) + align256(slots * d * 4)) : nullptr;
}

hipError_t launch_merge_for(const ta_plan* plan, int dtype, const AttnParams& p, int32_t d, hipStream_t st) {
  if (plan->merge.empty()) return hipSuccess;
  MergeParams m{};
  m.merge = reinterpret_cast<const MergeRow*>(static_cast<const unsigned char*>(plan->dev) + plan->layout.merge);
  m.part_acc = p.part_acc;
  m.part_ml = p.part_ml;
  m.o = p.o;
  m.lse = p.lse;
  m.n_rows = int32_t(plan->n_rows);
  m.n_merge = int32_t(plan->merge.size());
  m.hq = p.hq;
  return launch_merge(dtype, m, d, st);
}

}  // namespace
}  // namespace ta

using namespace ta;

extern "C" const char* tree_attn_version(void) { return "tree_attn 0.1 gfx950"; }

extern "C" int tree_attn_plan_info(const ta_plan* plan, ta_plan_info* out) try {
  if (!plan || !out) return fail(TA_ERR_INVALID_ARG, "plan_info: NULL argument");
  out->kind = plan->kind;
  out->n_pages = plan->n_pages;
  out->n_branches = plan->n_branches;
  out->n_work = int32_t(plan->work.size());
  out->n_rows = plan->n_rows;
  out->n_keys_a = plan->n_keys_a;
  out->n_keys_b = plan->n_keys_b;
  out->workspace_bytes = plan->layout.total;
  out->n_partials = plan->n_partials;
  out->visible_pairs = plan->visible_pairs;
  out->max_depth = plan->max_depth;
  return TA_OK;
} catch (...) {
  return ta::fail_exception("plan_info");
}

extern "C" int tree_attn_plan_export(const ta_plan* plan, int32_t field, int64_t* dst, int64_t cap,
                                     int64_t* n_written) try {
  if (!plan || !n_written) return fail(TA_ERR_INVALID_ARG, "plan_export: NULL argument");
  std::vector<int64_t> work_tmp;
  const std::vector<int64_t>* src = nullptr;
  const int k = plan->kind;
  switch (field) {
    case TA_FIELD_POSITION: if (k == TA_PLAN_PREFILL) src = &plan->position; break;
    case TA_FIELD_MAIN_END: if (k == TA_PLAN_PREFILL) src = &plan->main_end; break;
    case TA_FIELD_BRANCH_START: if (k == TA_PLAN_PREFILL) src = &plan->branch_start; break;
    case TA_FIELD_PAGES: if (k == TA_PLAN_PREFILL) src = &plan->pages5; break;
    case TA_FIELD_BRANCHES: if (k == TA_PLAN_PREFILL) src = &plan->branches3; break;
    case TA_FIELD_DECODE_ROWS: if (k == TA_PLAN_DECODE) src = &plan->decode_rows5; break;
    case TA_FIELD_VERIFY_MASK: if (k == TA_PLAN_VERIFY) src = &plan->verify_mask; break;
    case TA_FIELD_VERIFY_ROWS: if (k == TA_PLAN_VERIFY) src = &plan->verify_rows4; break;
    case TA_FIELD_BWD_WORK:
      if (k != TA_PLAN_PREFILL) break;
      for (const WorkItem& w : plan->kwork)
        work_tmp.insert(work_tmp.end(), {w.row0, w.nrows, w.a_lo, w.a_full, w.a_hi, w.b_lo, w.b_hi, w.out,
                                         w.flags, w.tile_lo, w.tile_hi, w.b_full});
      src = &work_tmp;
      break;
    case TA_FIELD_PAGED_TILES:
      if (plan->tile_a.empty() && plan->tile_b.empty()) break;
      work_tmp.assign(plan->tile_a.begin(), plan->tile_a.end());
      work_tmp.insert(work_tmp.end(), plan->tile_b.begin(), plan->tile_b.end());
      src = &work_tmp;
      break;
    case TA_FIELD_DEVICE_LAYOUT: {
      const DeviceLayout& L = plan->layout;
      work_tmp = {L.work, L.row_a, L.row_b, L.mask, L.merge, L.kwork, L.kmerge, L.trees, L.tile_a, L.tile_b, L.total};
      src = &work_tmp;
      break;
    }
    case TA_FIELD_DEVICE_IMAGE:
      work_tmp.resize(plan->blob.size() / sizeof(int64_t));
      if (!work_tmp.empty()) std::memcpy(work_tmp.data(), plan->blob.data(), work_tmp.size() * sizeof(int64_t));
      src = &work_tmp;
      break;
    case TA_FIELD_WORK:
      for (const WorkItem& w : plan->work)
        work_tmp.insert(work_tmp.end(), {w.row0, w.nrows, w.a_lo, w.a_full, w.a_hi, w.b_lo, w.b_hi, w.out,
                                         w.tile_lo, w.tile_hi, w.flags});
      src = &work_tmp;
      break;
    default: break;
  }
  if (!src) return fail(TA_ERR_INVALID_ARG, "plan_export: field not available for this plan kind");
  *n_written = int64_t(src->size());
  if (cap < int64_t(src->size())) return fail(TA_ERR_WORKSPACE, "plan_export: destination too small");
  if (!src->empty()) {
    if (!dst) return fail(TA_ERR_INVALID_ARG, "plan_export: dst is NULL");
    std::memcpy(dst, src->data(), src->size() * sizeof(int64_t));
  }
  return TA_OK;
} catch (...) {
  return ta::fail_exception("plan_export");
}

extern "C" int tree_attn_plan_upload(ta_plan* plan, void* dev_workspace, size_t bytes, void* stream) try {
  if (!plan) return fail(TA_ERR_INVALID_ARG, "plan_upload: plan is NULL");
  if (!dev_workspace) return fail(TA_ERR_WORKSPACE, "plan_upload: workspace is NULL");
  if (!aligned(dev_workspace, 256)) return fail(TA_ERR_INVALID_ARG, "plan_upload: workspace must be 256-byte aligned");
  if (int64_t(bytes) < plan->layout.total) return fail(TA_ERR_WORKSPACE, "plan_upload: workspace smaller than workspace_bytes");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (!plan->upload_event) {
    hipEvent_t ev = nullptr;
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return hip_status(e, "plan_upload");
    plan->upload_event = ev;
  }
  e = hipMemcpyAsync(dev_workspace, plan->blob.data(), plan->blob.size(), hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_status(e, "plan_upload");
  e = hipEventRecord(static_cast<hipEvent_t>(plan->upload_event), st);
  if (e != hipSuccess) return hip_status(e, "plan_upload");
  plan->dev = dev_workspace;
  return TA_OK;
} catch (...) {
  return ta::fail_exception("plan_upload");
}

extern "C" void tree_attn_plan_destroy(ta_plan* plan) {
  if (!plan) return;
  if (plan->upload_event) {
    // nothing to report from a destructor: a failed wait or release leaves
    // the error for the caller's next HIP call
    (void)hipEventSynchronize(static_cast<hipEvent_t>(plan->upload_event));
    (void)hipEventDestroy(static_cast<hipEvent_t>(plan->upload_event));
  }
  delete plan;
}

extern "C" int tree_attn_scratch_bytes(const ta_plan* plan, int32_t hq, int32_t head_dim, size_t* bytes) try {
  if (!plan || !bytes) return fail(TA_ERR_INVALID_ARG, "scratch_bytes: NULL argument");
  if (hq <= 0 || head_dim <= 0) return fail(TA_ERR_INVALID_ARG, "scratch_bytes: hq and head_dim must be positive");
  *bytes = size_t(scratch_need(plan, hq, head_dim));
  return TA_OK;
} catch (...) {
  return ta::fail_exception("scratch_bytes");
}

extern "C" int tree_attn_prefill(const ta_plan* plan, int32_t dtype, int32_t hq, int32_t hkv, int32_t head_dim,
                                 float scale, const void* q, const void* k, const void* v, void* o, float* lse,
                                 void* scratch, size_t scratch_bytes, void* stream) try {
  int rc = check_plan(plan, TA_PLAN_PREFILL, "prefill");
  if (rc) return rc;
  if ((rc = check_heads(dtype, hq, hkv, head_dim, scale))) return rc;
  const int64_t rows = plan->n_rows;
  if ((rc = check_tensor(q, rows, "q")) || (rc = check_tensor(k, rows, "k")) || (rc = check_tensor(v, rows, "v")) ||
      (rc = check_tensor(o, rows, "o")))
    return rc;
  if (lse && !aligned(lse, 4)) return fail(TA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if ((rc = check_scratch(plan, hq, head_dim, scratch, scratch_bytes, "prefill"))) return rc;
  if ((rc = check_uploaded(plan, "prefill"))) return rc;
  AttnParams p = base_params(plan, hq, hkv, scale);
  p.q = q;
  p.ka = p.kb = k;
  p.va = p.vb = v;
  p.o = o;
  p.lse = lse;
  set_partials(p, plan, hq, head_dim, scratch);
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = hip_status(launch_attention(kPrefill, dtype, p, int(plan->work.size()), head_dim, st), "prefill launch");
  if (rc) return rc;
  return hip_status(launch_merge_for(plan, dtype, p, head_dim, st), "prefill merge launch");
} catch (...) {
  return ta::fail_exception("prefill");
}

extern "C" int tree_attn_verify(const ta_plan* plan, int32_t dtype, int32_t hq, int32_t hkv, int32_t head_dim,
                                float scale, const void* q, const void* k_ctx, const void* v_ctx, const void* k_tree,
                                const void* v_tree, void* o, float* lse, void* scratch, size_t scratch_bytes,
                                void* stream) try {
  int rc = check_plan(plan, TA_PLAN_VERIFY, "verify");
  if (rc) return rc;
  if ((rc = check_heads(dtype, hq, hkv, head_dim, scale))) return rc;
  const int64_t rows = plan->n_rows;
  if ((rc = check_tensor(q, rows, "q")) || (rc = check_tensor(k_ctx, plan->n_keys_a, "k_ctx")) ||
      (rc = check_tensor(v_ctx, plan->n_keys_a, "v_ctx")) || (rc = check_tensor(k_tree, rows, "k_tree")) ||
      (rc = check_tensor(v_tree, rows, "v_tree")) || (rc = check_tensor(o, rows, "o")))
    return rc;
  if (lse && !aligned(lse, 4)) return fail(TA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if ((rc = check_scratch(plan, hq, head_dim, scratch, scratch_bytes, "verify"))) return rc;
  if ((rc = check_uploaded(plan, "verify"))) return rc;
  AttnParams p = base_params(plan, hq, hkv, scale);
  p.q = q;
  p.ka = k_ctx;
  p.va = v_ctx;
  p.kb = k_tree;
  p.vb = v_tree;
  p.o = o;
  p.lse = lse;
  set_partials(p, plan, hq, head_dim, scratch);
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = hip_status(launch_attention(kVerify, dtype, p, int(plan->work.size()), head_dim, st), "verify launch");
  if (rc) return rc;
  return hip_status(launch_merge_for(plan, dtype, p, head_dim, st), "verify merge launch");
} catch (...) {
  return ta::fail_exception("verify");
}

namespace {

int check_decode(const ta_plan* plan, int32_t dtype, int32_t hq, int32_t hkv, int32_t head_dim, float scale,
                 const void* q, const void* k_main, const void* v_main, const void* k_suffix, const void* v_suffix,
                 const void* o, const float* lse, const char* who) {
  int rc = check_plan(plan, TA_PLAN_DECODE, who);
  if (rc) return rc;
  if ((rc = check_heads(dtype, hq, hkv, head_dim, scale))) return rc;
  const int64_t rows = plan->n_rows;
  if ((rc = check_tensor(q, rows, "q")) || (rc = check_tensor(k_main, plan->n_keys_a, "k_main")) ||
      (rc = check_tensor(v_main, plan->n_keys_a, "v_main")) || (rc = check_tensor(k_suffix, plan->n_keys_b, "k_suffix")) ||
      (rc = check_tensor(v_suffix, plan->n_keys_b, "v_suffix")) || (rc = check_tensor(o, rows, "o")))
    return rc;
  if (lse && !aligned(lse, 4)) return fail(TA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  return TA_OK;
}

int launch_decode(const ta_plan* plan, int32_t dtype, int32_t hq, int32_t hkv, int32_t head_dim, float scale,
                  const void* q, const void* k_main, const void* v_main, const void* k_suffix, const void* v_suffix,
                  void* o, float* lse, void* scratch, void* stream) {
  AttnParams p = base_params(plan, hq, hkv, scale);
  p.q = q;
  p.ka = k_main;
  p.va = v_main;
  p.kb = k_suffix;
  p.vb = v_suffix;
  p.o = o;
  p.lse = lse;
  set_partials(p, plan, hq, head_dim, scratch);
  hipStream_t st = static_cast<hipStream_t>(stream);
  int rc = hip_status(launch_attention(kDecode, dtype, p, int(plan->work.size()), head_dim, st), "decode launch");
  if (rc) return rc;
  return hip_status(launch_merge_for(plan, dtype, p, head_dim, st), "decode merge launch");
}

}  // namespace

extern "C" int tree_attn_decode(const ta_plan* plan, int32_t dtype, int32_t hq, int32_t hkv, int32_t head_dim,
                                float scale, const void* q, const void* k_main, const void* v_main,
                                const void* k_suffix, const void* v_suffix, void* o, float* lse, void* scratch,
                                size_t scratch_bytes, void* stream) try {
  int rc = check_decode(plan, dtype, hq, hkv, head_dim, scale, q, k_main, v_main, k_suffix, v_suffix, o, lse,
                        "decode");
  if (rc) return rc;
  if ((rc = check_scratch(plan, hq, head_dim, scratch, scratch_bytes, "decode"))) return rc;
  if ((rc = check_uploaded(plan, "decode"))) return rc;
  return launch_decode(plan, dtype, hq, hkv, head_dim, scale, q, k_main, v_main, k_suffix, v_suffix, o, lse,
                       scratch, stream);
} catch (...) {
  return ta::fail_exception("decode");
}

extern "C" int tree_attn_decode_noalloc(const ta_plan* plan, int32_t dtype, int32_t hq, int32_t hkv,
                                        int32_t head_dim, float scale, const void* q, const void* k_main,
                                        const void* v_main, const void* k_suffix, const void* v_suffix, void* o,
                                        float* lse, void* stream) try {
  int rc = check_decode(plan, dtype, hq, hkv, head_dim, scale, q, k_main, v_main, k_suffix, v_suffix, o, lse,
                        "decode_noalloc");
  if (rc) return rc;
  const int64_t need = scratch_need(plan, hq, head_dim);
  if (need > int64_t(TA_STATIC_SCRATCH_BYTES))
    return fail(TA_ERR_CAPACITY, "decode_noalloc: the plan needs " + std::to_string(need) +
                                     " bytes of scratch; the static scratch holds " +
                                     std::to_string(int64_t(TA_STATIC_SCRATCH_BYTES)) + " (use tree_attn_decode)");
  if ((rc = check_uploaded(plan, "decode_noalloc"))) return rc;
  void* scratch = nullptr;
  if (need > 0 && (rc = hip_status(static_scratch(&scratch), "decode_noalloc: static scratch"))) return rc;
  return launch_decode(plan, dtype, hq, hkv, head_dim, scale, q, k_main, v_main, k_suffix, v_suffix, o, lse,
                       scratch, stream);
} catch (...) {
  return ta::fail_exception("decode_noalloc");
}

namespace {

// fp32 partial dK, dV of the split key tiles: [slots, hkv, 2, 64 keys, d]
int64_t kpart_bytes(const ta_plan* plan, int64_t hkv, int64_t head_dim) {
  return plan->n_kpart * hkv * 2 * kKeyTile * head_dim * 4;
}

}  // namespace

extern "C" int tree_attn_backward_scratch_bytes(const ta_plan* plan, int32_t hq, size_t* bytes) try {
  if (!plan || !bytes) return fail(TA_ERR_INVALID_ARG, "backward_scratch_bytes: NULL argument");
  if (hq <= 0) return fail(TA_ERR_INVALID_ARG, "backward_scratch_bytes: hq must be positive");
  // the partials are sized for the largest call: Hkv <= Hq, head_dim <= 128
  *bytes = size_t(2 * align256(plan->n_rows * hq * 4) + kpart_bytes(plan, hq, 128));
  return TA_OK;
} catch (...) {
  return ta::fail_exception("backward_scratch_bytes");
}

extern "C" int tree_attn_prefill_backward(const ta_plan* plan, int32_t dtype, int32_t hq, int32_t hkv,
                                          int32_t head_dim, float scale, const void* q, const void* k, const void* v,
                                          const void* o, const float* lse, const void* d_o, void* dq, void* dk,
                                          void* dv, void* scratch, size_t scratch_bytes, void* stream) try {
  int rc = check_plan(plan, TA_PLAN_PREFILL, "prefill_backward");
  if (rc) return rc;
  if ((rc = check_heads(dtype, hq, hkv, head_dim, scale))) return rc;
  if (dtype != TA_DTYPE_BF16) return fail(TA_ERR_UNSUPPORTED, "prefill_backward: only TA_DTYPE_BF16 is built");
  if (plan->n_partials > 0) return fail(TA_ERR_STATE, "prefill_backward: the plan is balanced; build an unbalanced one");
  const int64_t rows = plan->n_rows;
  if ((rc = check_tensor(q, rows, "q")) || (rc = check_tensor(k, rows, "k")) || (rc = check_tensor(v, rows, "v")) ||
      (rc = check_tensor(o, rows, "o")) || (rc = check_tensor(d_o, rows, "d_o")) || (rc = check_tensor(dq, rows, "dq")) ||
      (rc = check_tensor(dk, rows, "dk")) || (rc = check_tensor(dv, rows, "dv")))
    return rc;
  if (rows > 0 && !lse) return fail(TA_ERR_INVALID_ARG, "prefill_backward: lse is NULL");
  if (lse && !aligned(lse, 4)) return fail(TA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  const int64_t half = align256(rows * hq * 4);
  if (rows > 0) {
    if (!scratch) return fail(TA_ERR_WORKSPACE, "prefill_backward: scratch is NULL");
    if (!aligned(scratch, 256)) return fail(TA_ERR_INVALID_ARG, "prefill_backward: scratch must be 256-byte aligned");
    if (int64_t(scratch_bytes) < 2 * half + kpart_bytes(plan, hkv, head_dim))
      return fail(TA_ERR_WORKSPACE, "prefill_backward: scratch smaller than tree_attn_backward_scratch_bytes");
  }
  if ((rc = check_uploaded(plan, "prefill_backward"))) return rc;
  if (rows == 0) return TA_OK;
  const unsigned char* dev = static_cast<const unsigned char*>(plan->dev);
  BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dO = d_o;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.lse = lse;
  p.l2 = static_cast<float*>(scratch);
  p.dd = reinterpret_cast<float*>(static_cast<unsigned char*>(scratch) + half);
  p.work = reinterpret_cast<const WorkItem*>(dev + plan->layout.work);
  p.kwork = reinterpret_cast<const WorkItem*>(dev + plan->layout.kwork);
  p.kmerge = reinterpret_cast<const KMerge*>(dev + plan->layout.kmerge);
  p.kpart = reinterpret_cast<float*>(static_cast<unsigned char*>(scratch) + 2 * half);
  p.row_a = reinterpret_cast<const int32_t*>(dev + plan->layout.row_a);
  p.row_b = reinterpret_cast<const int32_t*>(dev + plan->layout.row_b);
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  p.c = scale * 1.4426950408889634f;
  p.scale = scale;
  p.n_rows = rows;
  return hip_status(launch_backward(p, int(plan->work.size()), int(plan->kwork.size()), int(plan->kmerge.size()),
                                    head_dim, static_cast<hipStream_t>(stream)),
                    "prefill_backward launch");
} catch (...) {
  return ta::fail_exception("prefill_backward");
}

namespace ta {
namespace {

// Argmax pieces per logits row: enough workgroups to fill the chip (about
// eight per compute unit) without cutting a row below 8192 entries.
constexpr int64_t kAcceptTargetBlocks = 2048;
constexpr int64_t kAcceptMinChunk = 8192;

void accept_geometry(int64_t rows, int64_t vocab, int32_t* chunks, int64_t* chunk_elems) {
  int64_t c = rows > 0 ? (kAcceptTargetBlocks + rows - 1) / rows : 1;
  c = std::max<int64_t>(1, std::min(c, (vocab + kAcceptMinChunk - 1) / kAcceptMinChunk));
  int64_t ce = (vocab + c - 1) / c;
  ce = (ce + 7) & ~int64_t(7);
  *chunk_elems = std::max<int64_t>(ce, 8);
  *chunks = int32_t(std::max<int64_t>(1, (vocab + *chunk_elems - 1) / *chunk_elems));
}

int64_t accept_rows(const ta_plan* plan) { return plan->n_rows + plan->n_branches; }

}  // namespace
}  // namespace ta

extern "C" int tree_attn_accept_scratch_bytes(const ta_plan* plan, int64_t vocab, size_t* bytes) try {
  if (!plan || !bytes) return fail(TA_ERR_INVALID_ARG, "accept_scratch_bytes: NULL argument");
  if (plan->kind != TA_PLAN_VERIFY) return fail(TA_ERR_STATE, "accept_scratch_bytes: needs a verify plan");
  if (vocab < 1 || vocab > INT32_MAX) return fail(TA_ERR_INVALID_ARG, "accept_scratch_bytes: vocab must be in [1, 2^31)");
  int32_t chunks;
  int64_t ce;
  const int64_t rows = accept_rows(plan);
  accept_geometry(rows, vocab, &chunks, &ce);
  *bytes = size_t(2 * align256(rows * chunks * 4));
  return TA_OK;
} catch (...) {
  return ta::fail_exception("accept_scratch_bytes");
}

extern "C" int tree_attn_accept(const ta_plan* plan, int32_t dtype, const void* logits, int64_t vocab, int64_t ld,
                                const int32_t* tokens, double tau, int32_t mode, int32_t* path, int32_t* n_path,
                                int32_t* next_token, void* scratch, size_t scratch_bytes, void* stream) try {
  int rc = check_plan(plan, TA_PLAN_VERIFY, "accept");
  if (rc) return rc;
  if (dtype != TA_DTYPE_BF16 && dtype != TA_DTYPE_F32)
    return fail(TA_ERR_UNSUPPORTED, "accept: dtype must be TA_DTYPE_BF16 or TA_DTYPE_F32");
  if (mode != TA_ACCEPT_TAU && mode != TA_ACCEPT_EXACT) return fail(TA_ERR_INVALID_ARG, "accept: unknown mode");
  if (mode == TA_ACCEPT_TAU && !(tau > 0.0 && std::isfinite(tau)))
    return fail(TA_ERR_INVALID_ARG, "accept: tau must be positive and finite");
  if (vocab < 1 || vocab > INT32_MAX) return fail(TA_ERR_INVALID_ARG, "accept: vocab must be in [1, 2^31)");
  if (ld < vocab) return fail(TA_ERR_INVALID_ARG, "accept: ld must be >= vocab");
  const int64_t rows = accept_rows(plan);
  const int64_t nodes = plan->n_rows;
  const size_t es = dtype == TA_DTYPE_BF16 ? 2 : 4;
  if (rows > 0 && (!logits || !aligned(logits, es)))
    return fail(TA_ERR_INVALID_ARG, "accept: logits is NULL or not aligned to its element size");
  if (nodes > 0 && (!tokens || !path)) return fail(TA_ERR_INVALID_ARG, "accept: tokens or path is NULL");
  if (plan->n_branches > 0 && (!n_path || !next_token))
    return fail(TA_ERR_INVALID_ARG, "accept: n_path or next_token is NULL");
  int32_t chunks;
  int64_t ce;
  accept_geometry(rows, vocab, &chunks, &ce);
  if (rows * chunks >= (int64_t(1) << 24)) return fail(TA_ERR_CAPACITY, "accept: too many logits rows for one launch");
  const int64_t half = align256(rows * chunks * 4);
  if (rows > 0) {
    if (!scratch) return fail(TA_ERR_WORKSPACE, "accept: scratch is NULL");
    if (!aligned(scratch, 256)) return fail(TA_ERR_INVALID_ARG, "accept: scratch must be 256-byte aligned");
    if (int64_t(scratch_bytes) < 2 * half)
      return fail(TA_ERR_WORKSPACE, "accept: scratch smaller than tree_attn_accept_scratch_bytes");
  }
  if ((rc = check_uploaded(plan, "accept"))) return rc;
  if (plan->n_branches == 0) return TA_OK;
  AcceptParams p{};
  p.logits = logits;
  p.ld = ld;
  p.vocab = vocab;
  p.tree_tab = reinterpret_cast<const int32_t*>(static_cast<const unsigned char*>(plan->dev) + plan->layout.trees);
  p.tokens = tokens;
  p.n_trees = plan->n_branches;
  p.exact = mode == TA_ACCEPT_EXACT;
  p.chunks = chunks;
  p.chunk_elems = ce;
  p.part_max = static_cast<float*>(scratch);
  p.part_idx = reinterpret_cast<int32_t*>(static_cast<unsigned char*>(scratch) + half);
  p.log_tau = mode == TA_ACCEPT_TAU ? std::log(tau) : 0.0;
  p.path = path;
  p.n_path = n_path;
  p.next_token = next_token;
  return hip_status(launch_accept(dtype, p, rows, static_cast<hipStream_t>(stream)), "accept launch");
} catch (...) {
  return ta::fail_exception("accept");
}

extern "C" int tree_attn_calib_mfma(int32_t blocks, int32_t iters, uint32_t seed, float* sink, int64_t* flops,
                                    void* stream) try {
  if (blocks <= 0 || blocks > (1 << 20) || iters <= 0 || iters > (1 << 24))
    return fail(TA_ERR_INVALID_ARG, "calib_mfma: blocks must be in [1, 2^20] and iters in [1, 2^24]");
  if (!sink || !aligned(sink, 4) || !flops) return fail(TA_ERR_INVALID_ARG, "calib_mfma: NULL or misaligned argument");
  *flops = calib_mfma_flops(blocks, iters);
  return hip_status(launch_calib_mfma(blocks, iters, seed, sink, static_cast<hipStream_t>(stream)), "calib_mfma launch");
} catch (...) {
  return ta::fail_exception("calib_mfma");
}

extern "C" int tree_attn_calib_read(const void* src, int64_t bytes, int32_t blocks, uint32_t* sink,
                                    void* stream) try {
  if (!src || !aligned(src, 16) || bytes <= 0 || bytes % 16)
    return fail(TA_ERR_INVALID_ARG, "calib_read: src must be 16-byte aligned and bytes a positive multiple of 16");
  if (blocks <= 0 || blocks > (1 << 20) || !sink || !aligned(sink, 4))
    return fail(TA_ERR_INVALID_ARG, "calib_read: blocks must be in [1, 2^20] with a 4-byte aligned sink");
  return hip_status(launch_calib_read(src, bytes, blocks, sink, static_cast<hipStream_t>(stream)), "calib_read launch");
} catch (...) {
  return ta::fail_exception("calib_read");
}

extern "C" int tree_attn_calib_tile(int32_t variant, int32_t blocks, int32_t iters, uint32_t seed, const void* src,
                                    int64_t src_bytes, float* sink, int64_t* flops, void* stream) try {
  if (variant < 0 || variant > 2) return fail(TA_ERR_INVALID_ARG, "calib_tile: variant must be 0, 1 or 2");
  if (blocks <= 0 || blocks > (1 << 20) || iters <= 0 || iters > (1 << 24))
    return fail(TA_ERR_INVALID_ARG, "calib_tile: blocks must be in [1, 2^20] and iters in [1, 2^24]");
  if (!sink || !aligned(sink, 4) || !flops) return fail(TA_ERR_INVALID_ARG, "calib_tile: NULL or misaligned argument");
  if (variant == 2 && (!src || !aligned(src, 16) || src_bytes < calib_tile_min_bytes()))
    return fail(TA_ERR_INVALID_ARG, "calib_tile: variant 2 needs a 16-byte aligned src of at least " +
                                        std::to_string(calib_tile_min_bytes()) + " bytes");
  *flops = calib_tile_flops(blocks, iters);
  return hip_status(launch_calib_tile(variant, blocks, iters, seed, src, src_bytes, sink,
                                      static_cast<hipStream_t>(stream)),
                    "calib_tile launch");
} catch (...) {
  return ta::fail_exception("calib_tile");
}
