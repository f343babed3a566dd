// C ABI of the tree-attention library: argument checks, plan upload and
// kernel dispatch.  Every check runs before the first launch, so a rejected
// call writes nothing (Megatron-LM pull request 7387, section "Summary":
// unsupported modes are rejected instead of silently ignored).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <functional>
#include <memory>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/tree_attn.h"
#include "fragments.hpp"
#include "kernel_common.hpp"
#include "plan.hpp"

namespace tree_attn {

template <typename T, int D, int HG>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
template <typename T, int D>
hipError_t launch_bwd_rowstat(const BwdArgs& a, hipStream_t stream);
template <typename T, int D>
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream);
template <typename T, int D, int HG>
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
hipError_t launch_reset_counters(ItemCounters* c, int n, hipStream_t stream);
unsigned persistent_grid(unsigned n_items);

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(const char* what, hipError_t e) {
  return fail(TREE_ATTN_HIP_ERROR, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

// the message store of tree_attn_last_error, for the other translation units
int report_error(int code, const std::string& msg) { return fail(code, msg); }

// Runs a host-side body so that no C++ exception crosses the C ABI: a failed
// host allocation (or any other exception) becomes TREE_ATTN_HIP_ERROR.
int guard_host(const char* fn, const std::function<int()>& body) noexcept {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return fail(TREE_ATTN_HIP_ERROR, std::string(fn) + ": out of host memory");
  } catch (const std::exception& e) {
    return fail(TREE_ATTN_HIP_ERROR, std::string(fn) + ": " + e.what());
  } catch (...) {
    return fail(TREE_ATTN_HIP_ERROR, std::string(fn) + ": unexpected host error");
  }
}

struct DevicePlan {
  int device = -1;
  void* block = nullptr;   // one allocation holding every table below
  void* staged = nullptr;  // pinned host copy of `block` (stream-ordered uploads only)
  Span* spans = nullptr;
  QTile* qtiles[kNumQTileSizes] = {};
  KTile* ktiles = nullptr;
  KTile* ktiles_wide = nullptr;
};

}  // namespace tree_attn

struct tree_attn_fragments_s {
  tree_attn::Fragments f;
};

struct tree_attn_plan_s {
  tree_attn::HostPlan host;
  tree_attn::DevicePlan dev;
  bool on_device = false;
};

using namespace tree_attn;

namespace {

void free_device(DevicePlan& d) {
  if (d.device < 0) return;
  int prev = -1;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(d.device);
  (void)hipFree(d.block);
  if (d.staged) (void)hipHostFree(d.staged);
  if (prev >= 0) (void)hipSetDevice(prev);
  d = DevicePlan{};
}

size_t align16(size_t n) { return (n + 15) & ~size_t(15); }

// Packs every table into one host staging buffer and uploads it with one
// allocation and one copy: synchronous (pageable staging) when `stream` is
// nullptr, otherwise ordered on *stream from pinned staging that the plan
// keeps until it is destroyed, so the host never waits for the device.
hipError_t upload_plan(const HostPlan& h, DevicePlan& d, const hipStream_t* stream) {
  struct Part {
    const void* src;
    size_t bytes;
    void** dst;
  };
  Part parts[3 + kNumQTileSizes] = {
      {h.spans.data(), h.spans.size() * sizeof(Span), reinterpret_cast<void**>(&d.spans)},
      {h.ktiles.data(), h.ktiles.size() * sizeof(KTile), reinterpret_cast<void**>(&d.ktiles)},
      {h.ktiles_wide.data(), h.ktiles_wide.size() * sizeof(KTile), reinterpret_cast<void**>(&d.ktiles_wide)},
  };
  for (int t = 0; t < kNumQTileSizes; ++t)
    parts[3 + t] = {h.qtiles[t].data(), h.qtiles[t].size() * sizeof(QTile), reinterpret_cast<void**>(&d.qtiles[t])};
  size_t total = 0;
  for (const Part& p : parts) total += align16(p.bytes);
  std::vector<unsigned char> pageable;
  unsigned char* stage = nullptr;
  if (stream) {
    hipError_t e = hipHostMalloc(&d.staged, std::max<size_t>(total, 16), hipHostMallocDefault);
    if (e != hipSuccess) return e;
    stage = static_cast<unsigned char*>(d.staged);
  } else {
    pageable.resize(total);
    stage = pageable.data();
  }
  std::memset(stage, 0, total);
  size_t off = 0;
  for (const Part& p : parts) {
    if (p.bytes) std::memcpy(stage + off, p.src, p.bytes);
    off += align16(p.bytes);
  }
  hipError_t e = hipMalloc(&d.block, std::max<size_t>(total, 16));
  if (e != hipSuccess) return e;
  e = stream ? hipMemcpyAsync(d.block, stage, total, hipMemcpyHostToDevice, *stream)
             : hipMemcpy(d.block, stage, total, hipMemcpyHostToDevice);
  off = 0;
  for (const Part& p : parts) {
    *p.dst = static_cast<unsigned char*>(d.block) + off;
    off += align16(p.bytes);
  }
  return e;
}

int make_plan(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len, int32_t num_segments,
              int32_t q_begin, int32_t q_end, tree_attn_plan_t* out, bool device,
              const hipStream_t* stream = nullptr) {
  if (!out) return fail(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_plan: out is NULL");
  *out = nullptr;
  return guard_host("tree_attn_plan", [&]() -> int {
    auto p = std::make_unique<tree_attn_plan_s>();
    std::string err;
    if (!build_host_plan(parent, seg_start, seg_len, num_segments, q_begin, q_end, p->host, err))
      return fail(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_plan: " + err);
    if (device) {
      hipError_t e = hipGetDevice(&p->dev.device);
      if (e == hipSuccess) e = upload_plan(p->host, p->dev, stream);
      if (e != hipSuccess) {
        free_device(p->dev);
        return hip_fail("tree_attn_plan: device upload", e);
      }
      p->on_device = true;
    }
    *out = p.release();
    return TREE_ATTN_OK;
  });
}

int gcd(int a, int b) {
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// Query tile of the forward and dQ kernels: 32 query rows per wavefront,
// HG heads of a key/value group side by side; 8 wavefronts per workgroup,
// 12 in the forward for bf16 rows of 128 with head groups of 4.
int fwd_query_tile(int hg, const tree_attn_shape* shape) {
  const bool twelve = hg == 4 && shape->dtype == TREE_ATTN_BF16 && shape->head_dim == 128;
  return 32 * ((twelve ? 12 : 8) / hg);
}
int dq_query_tile(int hg) { return 32 * (8 / hg); }

// Shared argument checks of fwd/bwd.  Returns 0 or an error code.
int check_call(const char* fn, tree_attn_plan_t plan, const tree_attn_shape* shape, float* scale_out) {
  const std::string f(fn);
  if (!plan) return fail(TREE_ATTN_INVALID_ARGUMENT, f + ": plan is NULL");
  if (!shape) return fail(TREE_ATTN_INVALID_ARGUMENT, f + ": shape is NULL");
  if (!plan->on_device) return fail(TREE_ATTN_INVALID_ARGUMENT, f + ": plan was built host-only");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->dev.device)
    return fail(TREE_ATTN_INVALID_ARGUMENT, f + ": plan was built on another device");
  if (shape->total_tokens != plan->host.T)
    return fail(TREE_ATTN_INVALID_ARGUMENT, f + ": shape.total_tokens " + std::to_string(shape->total_tokens) +
                                                " != plan tokens " + std::to_string(plan->host.T));
  if (shape->num_q_heads < 1 || shape->num_kv_heads < 1)
    return fail(TREE_ATTN_INVALID_ARGUMENT, f + ": head counts must be >= 1");
  if (shape->num_q_heads % shape->num_kv_heads != 0)
    return fail(TREE_ATTN_UNSUPPORTED, f + ": num_q_heads must be a multiple of num_kv_heads");
  if (shape->dtype == TREE_ATTN_BF16) {
    if (shape->head_dim != 128 && shape->head_dim != 64)
      return fail(TREE_ATTN_UNSUPPORTED, f + ": bf16 needs head_dim 64 or 128");
  } else if (shape->dtype == TREE_ATTN_FP32) {
    if (shape->head_dim != 64) return fail(TREE_ATTN_UNSUPPORTED, f + ": fp32 needs head_dim 64");
  } else {
    return fail(TREE_ATTN_UNSUPPORTED, f + ": dtype must be TREE_ATTN_BF16 or TREE_ATTN_FP32");
  }
  const int64_t rows = int64_t(shape->total_tokens) * shape->num_q_heads;
  if (rows * shape->head_dim >= (int64_t(1) << 31))
    return fail(TREE_ATTN_UNSUPPORTED, f + ": tensors are limited to 2^31 elements");
  // the query-major kernels gather K/V rows with 32-bit byte offsets
  const int64_t elem = shape->dtype == TREE_ATTN_BF16 ? 2 : 4;
  if (int64_t(shape->total_tokens) * shape->num_kv_heads * shape->head_dim * elem >= (int64_t(1) << 32))
    return fail(TREE_ATTN_UNSUPPORTED, f + ": k and v are limited to 2^32 bytes");
  const int hg = gcd(shape->num_q_heads / shape->num_kv_heads, 4);
  int64_t grid_q = 0;
  for (int tq : {fwd_query_tile(hg, shape), dq_query_tile(hg)})
    grid_q = std::max(grid_q, int64_t(plan->host.qtiles[qtile_index(tq)].size()) * (shape->num_q_heads / hg));
  const int64_t grid_k = int64_t(plan->host.ktiles.size()) * shape->num_kv_heads;  // >= the wide list's
  if (grid_q >= (int64_t(1) << 31) || grid_k >= (int64_t(1) << 31))
    return fail(TREE_ATTN_UNSUPPORTED, f + ": launch grid too large");
  // NaN and infinities are rejected; zero or a negative value asks for the default
  float s = shape->softmax_scale;
  if (!std::isfinite(s)) return fail(TREE_ATTN_INVALID_ARGUMENT, f + ": softmax_scale is not finite");
  if (s <= 0.f) s = 1.f / std::sqrt(float(shape->head_dim));
  *scale_out = s;
  return TREE_ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// the first four int32 fields of each 32-byte tile record (the rest hold
// what the kernels need with the tile: a first span, a segment end)
template <class Tile>
int export_heads(const std::vector<Tile>& tiles, int32_t* buf, int64_t cap, int64_t* count) {
  static_assert(sizeof(Tile) == 8 * sizeof(int32_t), "32-byte tile records");
  const int64_t n = int64_t(tiles.size()) * 4;
  *count = n;
  if (buf) {
    if (cap < n) return fail(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_plan_export: buffer too small");
    for (size_t i = 0; i < tiles.size(); ++i) std::memcpy(buf + 4 * i, &tiles[i], 4 * sizeof(int32_t));
  }
  return TREE_ATTN_OK;
}

}  // namespace

extern "C" {

int tree_attn_plan(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len, int32_t num_segments,
                   tree_attn_plan_t* out) {
  return make_plan(parent, seg_start, seg_len, num_segments, 0, -1, out, true);
}

int tree_attn_plan_async(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                         int32_t num_segments, void* stream, tree_attn_plan_t* out) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return make_plan(parent, seg_start, seg_len, num_segments, 0, -1, out, true, &s);
}

int tree_attn_plan_query_run(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                             int32_t num_segments, int32_t q_begin, int32_t q_end, tree_attn_plan_t* out) {
  return make_plan(parent, seg_start, seg_len, num_segments, q_begin, q_end, out, true);
}

int tree_attn_plan_query_run_host(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                                  int32_t num_segments, int32_t q_begin, int32_t q_end, tree_attn_plan_t* out) {
  return make_plan(parent, seg_start, seg_len, num_segments, q_begin, q_end, out, false);
}

int tree_attn_plan_host(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                        int32_t num_segments, tree_attn_plan_t* out) {
  return make_plan(parent, seg_start, seg_len, num_segments, 0, -1, out, false);
}

int tree_attn_fragment(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len, int32_t num_segments,
                       int32_t max_tokens, tree_attn_fragments_t* out) {
  if (!out) return fail(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_fragment: out is NULL");
  *out = nullptr;
  return guard_host("tree_attn_fragment", [&]() -> int {
    auto r = std::make_unique<tree_attn_fragments_s>();
    std::string err;
    if (!build_fragments(parent, seg_start, seg_len, num_segments, max_tokens, r->f, err))
      return fail(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_fragment: " + err);
    *out = r.release();
    return TREE_ATTN_OK;
  });
}

int tree_attn_fragments_destroy(tree_attn_fragments_t fr) {
  delete fr;
  return TREE_ATTN_OK;
}

int tree_attn_fragments_info(tree_attn_fragments_t fr, tree_attn_fragments_info_t* info) {
  if (!fr || !info) return fail(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_fragments_info: NULL argument");
  const Fragments& f = fr->f;
  info->num_fragments = int32_t(f.frag_seg_ptr.size()) - 1;
  info->num_segments = int32_t(f.seg_len.size());
  info->max_tokens = f.max_tokens;
  info->source_tokens = f.source_tokens;
  info->fragment_tokens = int64_t(f.token_source.size());
  return TREE_ATTN_OK;
}

int tree_attn_fragments_export(tree_attn_fragments_t fr, int32_t which, int32_t* buf, int64_t cap, int64_t* count) {
  if (!fr || !count) return fail(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_fragments_export: NULL argument");
  const Fragments& f = fr->f;
  const std::vector<int32_t>* src = nullptr;
  switch (which) {
    case TREE_ATTN_FRAG_SEG_PTR: src = &f.frag_seg_ptr; break;
    case TREE_ATTN_FRAG_TOKEN_PTR: src = &f.frag_token_ptr; break;
    case TREE_ATTN_FRAG_SEG_PARENT: src = &f.seg_parent; break;
    case TREE_ATTN_FRAG_SEG_LEN: src = &f.seg_len; break;
    case TREE_ATTN_FRAG_TOKEN_SOURCE: src = &f.token_source; break;
    case TREE_ATTN_FRAG_TOKEN_OWNER: src = &f.token_owner; break;
    default: return fail(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_fragments_export: unknown table");
  }
  *count = int64_t(src->size());
  if (!buf) return TREE_ATTN_OK;
  if (cap < *count) return fail(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_fragments_export: buffer too small");
  std::memcpy(buf, src->data(), src->size() * sizeof(int32_t));
  return TREE_ATTN_OK;
}

int tree_attn_plan_destroy(tree_attn_plan_t plan) {
  if (!plan) return TREE_ATTN_OK;
  free_device(plan->dev);
  delete plan;
  return TREE_ATTN_OK;
}

int tree_attn_plan_info(tree_attn_plan_t plan, tree_attn_plan_info_t* info) {
  if (!plan || !info) return fail(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_plan_info: NULL argument");
  const HostPlan& h = plan->host;
  info->total_tokens = h.T;
  info->num_segments = h.S;
  info->num_roots = h.num_roots;
  info->max_depth = h.max_depth;
  info->max_path_len = h.max_path;
  info->pairs = h.pairs;
  info->num_spans = int32_t(h.spans.size());
  info->num_q_tiles = int32_t(h.qtiles[0].size());
  info->num_kv_tiles = int32_t(h.ktiles.size());
  info->on_device = plan->on_device ? 1 : 0;
  info->q_begin = h.q_begin;
  info->q_end = h.q_end;
  return TREE_ATTN_OK;
}

int tree_attn_plan_export(tree_attn_plan_t plan, int32_t which, int32_t* buf, int64_t cap, int64_t* count) {
  if (!plan || !count) return fail(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_plan_export: NULL argument");
  const HostPlan& h = plan->host;
  const int32_t* src = nullptr;
  int64_t n = 0;
  switch (which) {
    case TREE_ATTN_EXPORT_SPAN_PTR:
      src = h.span_ptr.data();
      n = int64_t(h.span_ptr.size());
      break;
    case TREE_ATTN_EXPORT_SPANS:
      src = reinterpret_cast<const int32_t*>(h.spans.data());
      n = int64_t(h.spans.size()) * 4;
      break;
    case TREE_ATTN_EXPORT_Q_TILES:  // the first four fields of each record
      return export_heads(h.qtiles[0], buf, cap, count);
    case TREE_ATTN_EXPORT_KV_TILES:
      return export_heads(h.ktiles, buf, cap, count);
    case TREE_ATTN_EXPORT_SEG_DEPTH:
      src = h.depth.data();
      n = h.S;
      break;
    case TREE_ATTN_EXPORT_SEG_PREFIX:
      src = h.prefix.data();
      n = h.S;
      break;
    case TREE_ATTN_EXPORT_SEG_END:
      src = h.end.data();
      n = h.S;
      break;
    default:
      return fail(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_plan_export: unknown table " + std::to_string(which));
  }
  *count = n;
  if (buf) {
    if (cap < n) return fail(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_plan_export: buffer too small");
    if (n) std::memcpy(buf, src, size_t(n) * sizeof(int32_t));
  }
  return TREE_ATTN_OK;
}

static int run_fwd(const char* fn, const void* q, const void* k, const void* v, tree_attn_plan_t plan,
                   const tree_attn_shape* shape, void* out, float* lse, void* workspace, size_t workspace_bytes,
                   void* stream) {
  const std::string f(fn);
  float scale = 0.f;
  if (!q || !k || !v || !out || !lse) return fail(TREE_ATTN_INVALID_ARGUMENT, f + ": NULL tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(TREE_ATTN_INVALID_ARGUMENT, f + ": tensors must be 16-byte aligned");
  if (int rc = check_call(fn, plan, shape, &scale)) return rc;
  if (workspace) {
    if (!aligned16(workspace)) return fail(TREE_ATTN_INVALID_ARGUMENT, f + ": workspace must be 16-byte aligned");
    if (workspace_bytes < sizeof(ItemCounters))
      return fail(TREE_ATTN_INVALID_ARGUMENT, f + ": workspace " + std::to_string(workspace_bytes) +
                                                  " bytes < required " + std::to_string(sizeof(ItemCounters)));
  }
  const int G = shape->num_q_heads / shape->num_kv_heads;
  const int hg = gcd(G, 4);
  const int ti = qtile_index(fwd_query_tile(hg, shape));
  FwdArgs a;
  a.counters = static_cast<ItemCounters*>(workspace);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.tiles = plan->dev.qtiles[ti];
  a.spans = plan->dev.spans;
  a.n_tiles = int32_t(plan->host.qtiles[ti].size());
  a.T = shape->total_tokens;
  a.Hq = shape->num_q_heads;
  a.Hkv = shape->num_kv_heads;
  a.G = G;
  a.scale = scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  // the work-item counters start from zero whatever the workspace held
  if (a.counters) e = launch_reset_counters(a.counters, 1, s);
  if (e == hipSuccess) {
    if (shape->dtype == TREE_ATTN_BF16 && shape->head_dim == 128) {
      e = hg == 4 ? launch_fwd<__bf16, 128, 4>(a, s) : hg == 2 ? launch_fwd<__bf16, 128, 2>(a, s)
                                                             : launch_fwd<__bf16, 128, 1>(a, s);
    } else if (shape->dtype == TREE_ATTN_BF16) {
      e = hg == 4 ? launch_fwd<__bf16, 64, 4>(a, s) : hg == 2 ? launch_fwd<__bf16, 64, 2>(a, s)
                                                            : launch_fwd<__bf16, 64, 1>(a, s);
    } else {
      e = hg == 4 ? launch_fwd<float, 64, 4>(a, s) : hg == 2 ? launch_fwd<float, 64, 2>(a, s)
                                                           : launch_fwd<float, 64, 1>(a, s);
    }
  }
  if (e != hipSuccess) return hip_fail((f + ": launch").c_str(), e);
  return TREE_ATTN_OK;
}

int tree_attn_fwd(const void* q, const void* k, const void* v, tree_attn_plan_t plan, const tree_attn_shape* shape,
                  void* out, float* lse, void* stream) {
  return run_fwd("tree_attn_fwd", q, k, v, plan, shape, out, lse, nullptr, 0, stream);
}

size_t tree_attn_fwd_workspace_bytes(tree_attn_plan_t plan, const tree_attn_shape* shape) {
  if (!plan || !shape) return 0;
  return 256;
}

int tree_attn_fwd_ws(const void* q, const void* k, const void* v, tree_attn_plan_t plan, const tree_attn_shape* shape,
                     void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return fail(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_fwd_ws: workspace is NULL");
  return run_fwd("tree_attn_fwd_ws", q, k, v, plan, shape, out, lse, workspace, workspace_bytes, stream);
}

// workspace: -delta and -lse2 ([Hq, T] float32 each), then the work-item
// counters of the dK/dV and dQ passes
static size_t stats_bytes(const tree_attn_shape* shape) {
  const size_t bytes = 2 * size_t(shape->num_q_heads) * size_t(shape->total_tokens) * sizeof(float);
  return (bytes + 255) & ~size_t(255);
}

size_t tree_attn_bwd_workspace_bytes(tree_attn_plan_t plan, const tree_attn_shape* shape) {
  if (!plan || !shape || shape->total_tokens < 1 || shape->num_q_heads < 1) return 0;
  return stats_bytes(shape) + 2 * sizeof(ItemCounters);
}

}  // extern "C"

namespace {

enum Stage { kRowStat = 1, kDkDv = 2, kDq = 4, kAll = 7 };

// Checks shared by every backward entry point; fills `a` on success.
int prep_bwd(const char* fn, const void* q, const void* k, const void* v, const void* out, const float* lse,
             const void* dout, tree_attn_plan_t plan, const tree_attn_shape* shape, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes, int stages, BwdArgs& a, int& hg) {
  const std::string f(fn);
  float scale = 0.f;
  auto need = [&](const void* p, int st) { return (stages & st) && !p; };
  if (need(out, kRowStat) || need(dout, kAll) || need(q, kDkDv | kDq) || need(k, kDkDv | kDq) ||
      need(v, kDkDv | kDq) || need(lse, kAll) || need(dq, kDq) || need(dk, kDkDv) || need(dv, kDkDv) ||
      !workspace)
    return fail(TREE_ATTN_INVALID_ARGUMENT, f + ": NULL pointer");
  for (const void* p : {q, k, v, out, dout, static_cast<const void*>(dq), static_cast<const void*>(dk),
                        static_cast<const void*>(dv), static_cast<const void*>(workspace)})
    if (p && !aligned16(p)) return fail(TREE_ATTN_INVALID_ARGUMENT, f + ": pointers must be 16-byte aligned");
  if (int rc = check_call(fn, plan, shape, &scale)) return rc;
  const size_t ws = tree_attn_bwd_workspace_bytes(plan, shape);
  if (workspace_bytes < ws)
    return fail(TREE_ATTN_INVALID_ARGUMENT, f + ": workspace " + std::to_string(workspace_bytes) +
                                                " bytes < required " + std::to_string(ws));
  const int G = shape->num_q_heads / shape->num_kv_heads;
  hg = gcd(G, 4);
  const int ti = qtile_index(dq_query_tile(hg));
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = static_cast<float*>(workspace);
  a.counters = reinterpret_cast<ItemCounters*>(static_cast<char*>(workspace) + stats_bytes(shape));
  a.qtiles = plan->dev.qtiles[ti];
  // bf16 walks 128-key tiles, fp32 64-key tiles (its P hand-off is twice
  // as large, so wider tiles would not fit LDS)
  const bool wide = shape->dtype == TREE_ATTN_BF16;
  a.ktiles = wide ? plan->dev.ktiles_wide : plan->dev.ktiles;
  a.spans = plan->dev.spans;
  a.n_qtiles = int32_t(plan->host.qtiles[ti].size());
  a.n_ktiles = int32_t(wide ? plan->host.ktiles_wide.size() : plan->host.ktiles.size());
  a.T = shape->total_tokens;
  a.q_begin = plan->host.q_begin;
  a.q_end = plan->host.q_end;
  a.Hq = shape->num_q_heads;
  a.Hkv = shape->num_kv_heads;
  a.G = G;
  a.scale = scale;
  return TREE_ATTN_OK;
}

template <typename T, int D>
hipError_t launch_bwd_stages(const BwdArgs& a, int hg, int stages, hipStream_t s) {
  hipError_t e = hipSuccess;
  // the row-statistics stage zeroes both stages' counters; without it, a
  // stage zeroes its own first (a fresh workspace holds arbitrary bytes)
  if (!(stages & kRowStat) && (stages & kDkDv)) e = launch_reset_counters(&a.counters[0], 1, s);
  if (e == hipSuccess && !(stages & kRowStat) && (stages & kDq)) e = launch_reset_counters(&a.counters[1], 1, s);
  if (e == hipSuccess && (stages & kRowStat)) e = launch_bwd_rowstat<T, D>(a, s);
  if (e == hipSuccess && (stages & kDkDv)) e = launch_bwd_dkdv<T, D>(a, s);
  if (e == hipSuccess && (stages & kDq))
    e = hg == 4 ? launch_bwd_dq<T, D, 4>(a, s) : hg == 2 ? launch_bwd_dq<T, D, 2>(a, s) : launch_bwd_dq<T, D, 1>(a, s);
  return e;
}

int run_bwd(const char* fn, const BwdArgs& a, const tree_attn_shape* shape, int hg, int stages, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (shape->dtype == TREE_ATTN_BF16 && shape->head_dim == 128)
    e = launch_bwd_stages<__bf16, 128>(a, hg, stages, s);
  else if (shape->dtype == TREE_ATTN_BF16)
    e = launch_bwd_stages<__bf16, 64>(a, hg, stages, s);
  else
    e = launch_bwd_stages<float, 64>(a, hg, stages, s);
  if (e != hipSuccess) return hip_fail((std::string(fn) + ": launch").c_str(), e);
  return TREE_ATTN_OK;
}

}  // namespace

extern "C" {

int tree_attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse, const void* dout,
                  tree_attn_plan_t plan, const tree_attn_shape* shape, void* dq, void* dk, void* dv, void* workspace,
                  size_t workspace_bytes, void* stream) {
  BwdArgs a;
  int hg = 1;
  if (int rc = prep_bwd("tree_attn_bwd", q, k, v, out, lse, dout, plan, shape, dq, dk, dv, workspace,
                        workspace_bytes, kAll, a, hg))
    return rc;
  return run_bwd("tree_attn_bwd", a, shape, hg, kAll, stream);
}

int tree_attn_bwd_rowstat(const void* out, const float* lse, const void* dout, tree_attn_plan_t plan,
                          const tree_attn_shape* shape, void* workspace, size_t workspace_bytes, void* stream) {
  BwdArgs a;
  int hg = 1;
  if (int rc = prep_bwd("tree_attn_bwd_rowstat", nullptr, nullptr, nullptr, out, lse, dout, plan, shape,
                        nullptr, nullptr, nullptr, workspace, workspace_bytes, kRowStat, a, hg))
    return rc;
  return run_bwd("tree_attn_bwd_rowstat", a, shape, hg, kRowStat, stream);
}

int tree_attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                       tree_attn_plan_t plan, const tree_attn_shape* shape, void* dk, void* dv, void* workspace,
                       size_t workspace_bytes, void* stream) {
  BwdArgs a;
  int hg = 1;
  if (int rc = prep_bwd("tree_attn_bwd_dkdv", q, k, v, nullptr, lse, dout, plan, shape, nullptr, dk, dv,
                        workspace, workspace_bytes, kDkDv, a, hg))
    return rc;
  return run_bwd("tree_attn_bwd_dkdv", a, shape, hg, kDkDv, stream);
}

int tree_attn_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                     tree_attn_plan_t plan, const tree_attn_shape* shape, void* dq, void* workspace,
                     size_t workspace_bytes, void* stream) {
  BwdArgs a;
  int hg = 1;
  if (int rc = prep_bwd("tree_attn_bwd_dq", q, k, v, nullptr, lse, dout, plan, shape, dq, nullptr, nullptr,
                        workspace, workspace_bytes, kDq, a, hg))
    return rc;
  return run_bwd("tree_attn_bwd_dq", a, shape, hg, kDq, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free backward: the workspace lives in a fixed device array of
// this library.  Each GPU the library runs on holds its own copy of the
// array (its own address) until the process ends; host code reaches it only
// through the per-device address that hipGetSymbolAddress returns, never by
// the array's name (a host-side stand-in).

namespace {

constexpr size_t kScratchBytes = (size_t(64) << 20) + 256;  // row statistics of Hq * T <= 2^23 rows + counters
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_address(const char* fn, void** out) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return hip_fail(fn, e);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(TREE_ATTN_UNSUPPORTED, std::string(fn) + ": device index " + std::to_string(dev) + " >= 64");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess || !p)
      return hip_fail((std::string(fn) + ": hipGetSymbolAddress(scratch)").c_str(),
                      e != hipSuccess ? e : hipErrorInvalidSymbol);
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return TREE_ATTN_OK;
}

}  // namespace

extern "C" {

int tree_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* out, const float* lse,
                          const void* dout, tree_attn_plan_t plan, const tree_attn_shape* shape, void* dq, void* dk,
                          void* dv, void* stream) {
  const char* fn = "tree_attn_bwd_noalloc";
  if (plan && shape && shape->total_tokens >= 1 && shape->num_q_heads >= 1) {
    const size_t need = tree_attn_bwd_workspace_bytes(plan, shape);
    if (need > kScratchBytes)
      return fail(TREE_ATTN_UNSUPPORTED, std::string(fn) + ": the backward needs " + std::to_string(need) +
                                             " bytes of scratch (2 * Hq * T floats + counters), above the fixed " +
                                             std::to_string(kScratchBytes) + " (Hq * T <= 8,388,608)");
  }
  void* ws = nullptr;
  if (int rc = scratch_address(fn, &ws)) return rc;
  BwdArgs a;
  int hg = 1;
  // the row-statistics stage writes every statistic the later stages read
  // and zeroes their work counters, so nothing left by an earlier call is used
  if (int rc = prep_bwd(fn, q, k, v, out, lse, dout, plan, shape, dq, dk, dv, ws, kScratchBytes, kAll, a, hg))
    return rc;
  return run_bwd(fn, a, shape, hg, kAll, stream);
}

const char* tree_attn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
