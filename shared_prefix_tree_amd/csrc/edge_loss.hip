// Sampled-edge projection and loss: only the hidden states that are the
// source of a sampled token go through the vocabulary head, each sampled
// token (edge) owning its loss once (Megatron-LM pull request 7387, section
// "Summary": the edge-source hidden states are picked out before the
// vocabulary projection; issue "Shared-prefix training with context
// parallelism for exact agent trajectories", section "Describe the solution
// you'd like": only sampled-edge sources go through the vocabulary head, and
// each sampled action has a single loss owner).
//
// For edge e with source token src[e] and sampled token tgt[e]:
//   logits[e] = W h[src[e]]       (W: [V, d], h: [T, d], bf16)
//   lse[e]    = log sum_v exp(logits[e, v]),   loss[e] = lse[e] - logits[e, tgt[e]]
// and, given dloss[e], G[e, v] = (softmax(logits[e])_v - [v == tgt[e]]) dloss[e],
//   dh[t] = sum over edges e with src[e] = t of G[e] W   (0 for other rows)
//   dW    = sum_e G[e]^T h[src[e]].
//
// Pass structure (one GPU; a tensor-parallel rank would own a vocabulary
// slice and all-reduce the row statistics): gather the E source rows once,
// then walk the vocabulary in chunks of kVocabChunk rows.  Each chunk's
// logits are one library GEMM into an fp32 [E, chunk] buffer that never
// holds more than one chunk; our kernels fold them into running row
// statistics (forward) or turn them into G (backward), and two more library
// GEMMs accumulate dh (fp32, over chunks, in chunk order) and write the
// chunk's rows of dW.  dh is scattered back to the tokens by a per-token sum
// over that token's edges in edge order.  No atomics anywhere (the GEMMs run
// with rocBLAS atomics disabled), so results are bitwise reproducible.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <functional>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/tree_attn.h"
#include "edge_plan.hpp"

namespace tree_attn {
int report_error(int code, const std::string& msg);
int guard_host(const char* fn, const std::function<int()>& body) noexcept;
}

using tree_attn::report_error;

struct tree_attn_edges_s {
  int device = -1;
  int32_t E = 0, T = 0, V = 0;
  void* block = nullptr;        // src, tgt, row_ptr, edge ids (device, int32)
  int32_t* src = nullptr;       // [E]
  int32_t* tgt = nullptr;       // [E]
  int32_t* row_ptr = nullptr;   // [T + 1]: token t's edges are ids[row_ptr[t] .. row_ptr[t + 1])
  int32_t* ids = nullptr;       // [E] edge ids grouped by source token, ascending within a token
};

namespace {

constexpr int kVocabChunk = 8192;

__device__ inline float bf16_to_f32(unsigned short b) { return __uint_as_float(unsigned(b) << 16); }
__device__ inline unsigned short f32_to_bf16(float f) {  // round to nearest even
  const unsigned u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (unsigned short)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  return (unsigned short)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// hg[e] = h[src[e]]: one thread per 16-byte piece
__global__ void gather_rows_kernel(const uint4* __restrict__ h, const int32_t* __restrict__ src, int E, int pieces,
                                   uint4* __restrict__ hg) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)E * pieces) return;
  const int e = int(i / pieces), p = int(i % pieces);
  hg[i] = h[(long long)src[e] * pieces + p];
}

// One 256-thread block per edge row of a chunk.  Thread t holds columns
// 4 (t + 256 k) .. + 3 for k < kPer in registers, so a row is read from HBM
// once; columns past n read as -inf.  Rows are 16-byte aligned when the
// leading dimension is a multiple of 4 (every chunk but a vocabulary of
// fewer than kVocabChunk rows that is not), else the loads are scalar.
constexpr int kRowThreads = 256;
constexpr int kPer = kVocabChunk / (4 * kRowThreads);

__device__ inline void load_row(const float* __restrict__ row, int n, bool vec, float (&v)[kPer][4]) {
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int j = 4 * (threadIdx.x + kRowThreads * k);
    if (vec && j + 3 < n) {
      const float4 x = *reinterpret_cast<const float4*>(row + j);
      v[k][0] = x.x, v[k][1] = x.y, v[k][2] = x.z, v[k][3] = x.w;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) v[k][c] = j + c < n ? row[j + c] : -INFINITY;
    }
  }
}

// fixed-order block reduction (shuffle tree inside a wave, then the four
// wave results in order), so the result does not depend on scheduling
__device__ inline float block_reduce(float v, float* red, bool is_max) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float u = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = is_max ? fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))
                         : (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

// Running row statistics over one chunk: columns [c0, c0 + n) of the
// vocabulary, logits[e, j] at L[e * ld + j]
// Saved logits (optional): row e of chunk ci is kept as fp16 values of
// logit - cmax[e][ci], where cmax is the chunk's row maximum, so every kept
// value is <= 0 and the large probabilities keep fp16's relative precision.
struct Saved {
  __half* z;      // [E][V]
  float* cmax;    // [E][nchunks]
  int V, nchunks;
};

__global__ __launch_bounds__(kRowThreads) void chunk_stats_kernel(const float* __restrict__ L, int ld, int n, int c0,
                                                                  const int32_t* __restrict__ tgt,
                                                                  float* __restrict__ m, float* __restrict__ s,
                                                                  float* __restrict__ tl, int first, Saved sv,
                                                                  int ci) {
  __shared__ float red[kRowThreads / 64];
  const int e = blockIdx.x;
  const float* row = L + (long long)e * ld;
  float v[kPer][4];
  load_row(row, n, (ld & 3) == 0, v);
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < kPer; ++k)
#pragma unroll
    for (int c = 0; c < 4; ++c) mx = fmaxf(mx, v[k][c]);
  mx = block_reduce(mx, red, true);
  const float m_old = first ? -INFINITY : m[e];
  const float m_new = fmaxf(m_old, mx);
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < kPer; ++k)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc += __expf(v[k][c] - m_new);
  acc = block_reduce(acc, red, false);
  if (sv.z) {
    __half* zr = sv.z + (long long)e * sv.V + c0;
    const bool vec = ((sv.V & 3) == 0);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = 4 * (threadIdx.x + kRowThreads * k);
      if (vec && j + 3 < n) {
        const __half2 lo = __floats2half2_rn(v[k][0] - mx, v[k][1] - mx);
        const __half2 hi = __floats2half2_rn(v[k][2] - mx, v[k][3] - mx);
        uint2 pk;
        pk.x = *reinterpret_cast<const unsigned*>(&lo);
        pk.y = *reinterpret_cast<const unsigned*>(&hi);
        *reinterpret_cast<uint2*>(zr + j) = pk;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (j + c < n) zr[j + c] = __float2half_rn(v[k][c] - mx);
      }
    }
    if (threadIdx.x == 0) sv.cmax[(long long)e * sv.nchunks + ci] = mx;
  }
  if (threadIdx.x == 0) {
    const float s_old = first ? 0.f : s[e] * __expf(m_old - m_new);
    m[e] = m_new;
    s[e] = s_old + acc;
    const int t = tgt[e] - c0;
    if (t >= 0 && t < n) tl[e] = row[t];
  }
}

__global__ void finalize_kernel(const float* __restrict__ m, const float* __restrict__ s,
                                const float* __restrict__ tl, int E, float* __restrict__ loss,
                                float* __restrict__ lse) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const float l = m[e] + logf(s[e]);
  lse[e] = l;
  loss[e] = l - tl[e];
}

// G[e, j] = (exp(L[e, j] - lse[e]) - [c0 + j == tgt[e]]) dloss[e], bf16; one
// block per edge row, four columns per thread and step
__global__ __launch_bounds__(kRowThreads) void chunk_grad_kernel(const float* __restrict__ L, int ld, int n, int c0,
                                                                 const int32_t* __restrict__ tgt,
                                                                 const float* __restrict__ lse,
                                                                 const float* __restrict__ dloss,
                                                                 unsigned short* __restrict__ G) {
  const int e = blockIdx.x;
  const float* row = L + (long long)e * ld;
  unsigned short* grow = G + (long long)e * ld;
  const float le = lse[e], dl = dloss[e];
  const int t = tgt[e] - c0;
  const bool vec = (ld & 3) == 0;
  for (int j = 4 * threadIdx.x; j < n; j += 4 * kRowThreads) {
    float x[4];
    if (vec && j + 3 < n) {
      const float4 q = *reinterpret_cast<const float4*>(row + j);
      x[0] = q.x, x[1] = q.y, x[2] = q.z, x[3] = q.w;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) x[c] = j + c < n ? row[j + c] : 0.f;
    }
    unsigned short g[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) g[c] = f32_to_bf16((__expf(x[c] - le) - (j + c == t ? 1.f : 0.f)) * dl);
    if (vec && j + 3 < n) {
      *reinterpret_cast<uint2*>(grow + j) =
          make_uint2(unsigned(g[0]) | (unsigned(g[1]) << 16), unsigned(g[2]) | (unsigned(g[3]) << 16));
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (j + c < n) grow[j + c] = g[c];
    }
  }
}

// G from the saved logits: p = exp(z + cmax - lse)
__global__ __launch_bounds__(kRowThreads) void chunk_grad_saved_kernel(Saved sv, int ci, int ld, int n, int c0,
                                                                       const int32_t* __restrict__ tgt,
                                                                       const float* __restrict__ lse,
                                                                       const float* __restrict__ dloss,
                                                                       unsigned short* __restrict__ G) {
  const int e = blockIdx.x;
  const __half* zr = sv.z + (long long)e * sv.V + c0;
  unsigned short* grow = G + (long long)e * ld;
  const float off = sv.cmax[(long long)e * sv.nchunks + ci] - lse[e], dl = dloss[e];
  const int t = tgt[e] - c0;
  const bool vec = ((sv.V & 3) == 0) && ((ld & 3) == 0);
  for (int j = 4 * threadIdx.x; j < n; j += 4 * kRowThreads) {
    float x[4];
    if (vec && j + 3 < n) {
      const uint2 pk = *reinterpret_cast<const uint2*>(zr + j);
      const float2 lo = __half22float2(*reinterpret_cast<const __half2*>(&pk.x));
      const float2 hi = __half22float2(*reinterpret_cast<const __half2*>(&pk.y));
      x[0] = lo.x, x[1] = lo.y, x[2] = hi.x, x[3] = hi.y;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) x[c] = j + c < n ? __half2float(zr[j + c]) : 0.f;
    }
    unsigned short g[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) g[c] = f32_to_bf16((__expf(x[c] + off) - (j + c == t ? 1.f : 0.f)) * dl);
    if (vec && j + 3 < n) {
      *reinterpret_cast<uint2*>(grow + j) =
          make_uint2(unsigned(g[0]) | (unsigned(g[1]) << 16), unsigned(g[2]) | (unsigned(g[3]) << 16));
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (j + c < n) grow[j + c] = g[c];
    }
  }
}

// dh[t] = sum of dhg over t's edges, in edge order; 0 for tokens without
// one.  One thread per 8 columns of a token row (d is a multiple of 8).
__global__ void scatter_rows_kernel(const float* __restrict__ dhg, const int32_t* __restrict__ row_ptr,
                                    const int32_t* __restrict__ ids, int T, int d, uint4* __restrict__ dh) {
  const int pieces = d / 8;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)T * pieces) return;
  const int t = int(i / pieces), c = int(i % pieces) * 8;
  float acc[8] = {};
  for (int k = row_ptr[t]; k < row_ptr[t + 1]; ++k) {
    const float4* p = reinterpret_cast<const float4*>(dhg + (long long)ids[k] * d + c);
    const float4 x = p[0], y = p[1];
    acc[0] += x.x, acc[1] += x.y, acc[2] += x.z, acc[3] += x.w;
    acc[4] += y.x, acc[5] += y.y, acc[6] += y.z, acc[7] += y.w;
  }
  unsigned u[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) u[q] = unsigned(f32_to_bf16(acc[2 * q])) | (unsigned(f32_to_bf16(acc[2 * q + 1])) << 16);
  dh[i] = make_uint4(u[0], u[1], u[2], u[3]);
}

struct Handle {
  rocblas_handle h = nullptr;
};

std::mutex g_blas_mu;
Handle g_blas[64];

int blas_for(int dev, rocblas_handle* out) {
  if (dev < 0 || dev >= 64) return report_error(TREE_ATTN_HIP_ERROR, "edge loss: device index out of range");
  if (!g_blas[dev].h) {
    if (rocblas_create_handle(&g_blas[dev].h) != rocblas_status_success)
      return report_error(TREE_ATTN_HIP_ERROR, "edge loss: rocblas_create_handle failed");
    rocblas_set_atomics_mode(g_blas[dev].h, rocblas_atomics_not_allowed);
  }
  *out = g_blas[dev].h;
  return TREE_ATTN_OK;
}

// column-major GEMM, bf16 inputs, fp32 compute, output type `ct`
rocblas_status gemm(rocblas_handle h, rocblas_operation ta, rocblas_operation tb, int m, int n, int k,
                    const void* A, int lda, const void* B, int ldb, float beta, void* C, rocblas_datatype ct,
                    int ldc) {
  const float alpha = 1.f;
  return rocblas_gemm_ex(h, ta, tb, m, n, k, &alpha, A, rocblas_datatype_bf16_r, lda, B, rocblas_datatype_bf16_r,
                         ldb, &beta, C, ct, ldc, C, ct, ldc, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0,
                         0);
}

struct Workspace {
  unsigned short* hg;  // [E, d] bf16
  float* dhg;          // [E, d]
  float* L;            // [E, chunk]
  unsigned short* G;   // [E, chunk] bf16
  float *m, *s, *tl;   // [E]
};

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

size_t workspace_layout(int E, int d, int V, Workspace* w, char* base) {
  const int chunk = std::min(V, kVocabChunk);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  Workspace x;
  x.hg = reinterpret_cast<unsigned short*>(take(size_t(E) * d * 2));
  x.dhg = reinterpret_cast<float*>(take(size_t(E) * d * 4));
  x.L = reinterpret_cast<float*>(take(size_t(E) * chunk * 4));
  x.G = reinterpret_cast<unsigned short*>(take(size_t(E) * chunk * 2));
  x.m = reinterpret_cast<float*>(take(size_t(E) * 4));
  x.s = reinterpret_cast<float*>(take(size_t(E) * 4));
  x.tl = reinterpret_cast<float*>(take(size_t(E) * 4));
  if (w) *w = x;
  return off;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_call(const char* fn, tree_attn_edges_t edges, int32_t d, const void* a, const void* b, const void* c,
               const void* ws, size_t ws_bytes) {
  const std::string f(fn);
  if (!edges) return report_error(TREE_ATTN_INVALID_ARGUMENT, f + ": edges is NULL");
  if (!a || !b || !c || !ws) return report_error(TREE_ATTN_INVALID_ARGUMENT, f + ": NULL pointer");
  if (!aligned16(a) || !aligned16(b) || !aligned16(ws))
    return report_error(TREE_ATTN_INVALID_ARGUMENT, f + ": pointers must be 16-byte aligned");
  if (d < 8 || d % 8 != 0)
    return report_error(TREE_ATTN_UNSUPPORTED, f + ": hidden size must be a positive multiple of 8");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != edges->device)
    return report_error(TREE_ATTN_INVALID_ARGUMENT, f + ": edges were built on another device");
  const size_t need = tree_attn_edge_loss_workspace_bytes(edges, d);
  if (ws_bytes < need)
    return report_error(TREE_ATTN_INVALID_ARGUMENT, f + ": workspace " + std::to_string(ws_bytes) +
                                                        " bytes < required " + std::to_string(need));
  return TREE_ATTN_OK;
}

int hip_error(const char* fn, hipError_t e) {
  return report_error(TREE_ATTN_HIP_ERROR, std::string(fn) + ": " + hipGetErrorString(e));
}

int blas_error(const char* fn, rocblas_status st) {
  return report_error(TREE_ATTN_HIP_ERROR, std::string(fn) + ": rocBLAS status " + std::to_string(int(st)));
}

// logits of vocabulary rows [c0, c0 + n) for every edge into w.L ([E, chunk])
rocblas_status chunk_logits(rocblas_handle h, const Workspace& w, const void* W, int E, int d, int c0, int n,
                            int chunk) {
  // column-major: L^T [n, E] (ld chunk) = W_c^T-view ... W_c is row-major [n, d] = column-major [d, n]
  return gemm(h, rocblas_operation_transpose, rocblas_operation_none, n, E, d,
              static_cast<const unsigned short*>(W) + size_t(c0) * d, d, w.hg, d, 0.f, w.L,
              rocblas_datatype_f32_r, chunk);
}

}  // namespace

extern "C" {

int tree_attn_edges(const int32_t* edge_src, const int32_t* edge_tgt, int32_t num_edges, int32_t num_tokens,
                    int32_t vocab, tree_attn_edges_t* out) {
  if (!out) return report_error(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_edges: out is NULL");
  *out = nullptr;
  if (int64_t(num_edges) * kVocabChunk >= (int64_t(1) << 31))
    return report_error(TREE_ATTN_UNSUPPORTED, "tree_attn_edges: more than 262,143 edges");
  return tree_attn::guard_host("tree_attn_edges", [&]() -> int {
    // CSR by source token, edges ascending within a token
    std::vector<int32_t> row_ptr, ids;
    std::string err;
    if (!tree_attn::build_edge_csr(edge_src, edge_tgt, num_edges, num_tokens, vocab, row_ptr, ids, err))
      return report_error(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_edges: " + err);

    auto r = std::make_unique<tree_attn_edges_s>();
    r->E = num_edges;
    r->T = num_tokens;
    r->V = vocab;
    const size_t n_src = align256(size_t(num_edges) * 4), n_ptr = align256((size_t(num_tokens) + 1) * 4);
    const size_t total = 3 * n_src + n_ptr;
    std::vector<char> stage(total, 0);  // (host allocations before the device one: nothing leaks on a throw)
    std::memcpy(stage.data(), edge_src, size_t(num_edges) * 4);
    std::memcpy(stage.data() + n_src, edge_tgt, size_t(num_edges) * 4);
    std::memcpy(stage.data() + 2 * n_src, ids.data(), size_t(num_edges) * 4);
    std::memcpy(stage.data() + 3 * n_src, row_ptr.data(), row_ptr.size() * 4);
    hipError_t e = hipGetDevice(&r->device);
    if (e == hipSuccess) e = hipMalloc(&r->block, total);
    if (e != hipSuccess)
      return report_error(TREE_ATTN_HIP_ERROR, std::string("tree_attn_edges: ") + hipGetErrorString(e));
    char* b = static_cast<char*>(r->block);
    r->src = reinterpret_cast<int32_t*>(b);
    r->tgt = reinterpret_cast<int32_t*>(b + n_src);
    r->ids = reinterpret_cast<int32_t*>(b + 2 * n_src);
    r->row_ptr = reinterpret_cast<int32_t*>(b + 3 * n_src);
    e = hipMemcpy(r->block, stage.data(), total, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(r->block);
      return report_error(TREE_ATTN_HIP_ERROR, std::string("tree_attn_edges: upload: ") + hipGetErrorString(e));
    }
    *out = r.release();
    return TREE_ATTN_OK;
  });
}

int tree_attn_edges_destroy(tree_attn_edges_t edges) {
  if (!edges) return TREE_ATTN_OK;
  int prev = -1;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(edges->device);
  (void)hipFree(edges->block);
  if (prev >= 0) (void)hipSetDevice(prev);
  delete edges;
  return TREE_ATTN_OK;
}

size_t tree_attn_edge_loss_workspace_bytes(tree_attn_edges_t edges, int32_t hidden) {
  if (!edges || hidden < 1) return 0;
  return workspace_layout(edges->E, hidden, edges->V, nullptr, nullptr);
}

size_t tree_attn_edge_loss_saved_bytes(tree_attn_edges_t edges) {
  if (!edges) return 0;
  const int nch = (edges->V + kVocabChunk - 1) / kVocabChunk;
  return align256(size_t(edges->E) * edges->V * 2) + align256(size_t(edges->E) * nch * 4);
}

}  // extern "C"

namespace {

int saved_view(const char* fn, tree_attn_edges_t edges, void* saved, size_t saved_bytes, Saved* sv) {
  *sv = Saved{nullptr, nullptr, edges->V, (edges->V + kVocabChunk - 1) / kVocabChunk};
  if (!saved) return TREE_ATTN_OK;
  if (!aligned16(saved))
    return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": saved must be 16-byte aligned");
  if (saved_bytes < tree_attn_edge_loss_saved_bytes(edges))
    return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": saved buffer too small");
  sv->z = static_cast<__half*>(saved);
  sv->cmax = reinterpret_cast<float*>(static_cast<char*>(saved) + align256(size_t(edges->E) * edges->V * 2));
  return TREE_ATTN_OK;
}

}  // namespace

extern "C" {

int tree_attn_edge_loss_fwd(const void* hidden, const void* weight, int32_t d, tree_attn_edges_t edges, float* loss,
                            float* lse, void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                            void* stream) {
  const char* fn = "tree_attn_edge_loss_fwd";
  if (int rc = check_call(fn, edges, d, hidden, weight, loss, workspace, workspace_bytes)) return rc;
  if (!lse) return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": NULL pointer");
  Saved sv;
  if (int rc = saved_view(fn, edges, saved, saved_bytes, &sv)) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int E = edges->E, V = edges->V, chunk = std::min(V, kVocabChunk);
  Workspace w;
  workspace_layout(E, d, V, &w, static_cast<char*>(workspace));
  std::lock_guard<std::mutex> lock(g_blas_mu);
  rocblas_handle h;
  if (int rc = blas_for(edges->device, &h)) return rc;
  if (rocblas_status st = rocblas_set_stream(h, s); st != rocblas_status_success) return blas_error(fn, st);
  const int pieces = d / 8;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(unsigned((int64_t(E) * pieces + 255) / 256)), dim3(256), 0, s,
                     static_cast<const uint4*>(hidden), edges->src, E, pieces, reinterpret_cast<uint4*>(w.hg));
  for (int c0 = 0; c0 < V; c0 += chunk) {
    const int n = std::min(chunk, V - c0);
    if (rocblas_status st = chunk_logits(h, w, weight, E, d, c0, n, chunk); st != rocblas_status_success)
      return blas_error(fn, st);
    hipLaunchKernelGGL(chunk_stats_kernel, dim3(E), dim3(kRowThreads), 0, s, w.L, chunk, n, c0, edges->tgt, w.m, w.s,
                       w.tl, c0 == 0 ? 1 : 0, sv, c0 / kVocabChunk);
  }
  hipLaunchKernelGGL(finalize_kernel, dim3((E + 255) / 256), dim3(256), 0, s, w.m, w.s, w.tl, E, loss, lse);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return hip_error(fn, e);
  return TREE_ATTN_OK;
}

int tree_attn_edge_loss_bwd(const void* hidden, const void* weight, int32_t d, tree_attn_edges_t edges,
                            const float* lse, const void* saved, size_t saved_bytes, const float* dloss,
                            void* dhidden, void* dweight, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "tree_attn_edge_loss_bwd";
  if (int rc = check_call(fn, edges, d, hidden, weight, dhidden, workspace, workspace_bytes)) return rc;
  if (!lse || !dloss || !dweight) return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": NULL pointer");
  Saved sv;
  if (int rc = saved_view(fn, edges, const_cast<void*>(saved), saved_bytes, &sv)) return rc;
  if (!aligned16(dhidden) || !aligned16(dweight))
    return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int E = edges->E, V = edges->V, T = edges->T, chunk = std::min(V, kVocabChunk);
  Workspace w;
  workspace_layout(E, d, V, &w, static_cast<char*>(workspace));
  std::lock_guard<std::mutex> lock(g_blas_mu);
  rocblas_handle h;
  if (int rc = blas_for(edges->device, &h)) return rc;
  if (rocblas_status st = rocblas_set_stream(h, s); st != rocblas_status_success) return blas_error(fn, st);
  const int pieces = d / 8;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(unsigned((int64_t(E) * pieces + 255) / 256)), dim3(256), 0, s,
                     static_cast<const uint4*>(hidden), edges->src, E, pieces, reinterpret_cast<uint4*>(w.hg));
  for (int c0 = 0; c0 < V; c0 += chunk) {
    const int n = std::min(chunk, V - c0);
    if (sv.z) {  // the forward kept this chunk's logits
      hipLaunchKernelGGL(chunk_grad_saved_kernel, dim3(E), dim3(kRowThreads), 0, s, sv, c0 / kVocabChunk, chunk, n,
                         c0, edges->tgt, lse, dloss, w.G);
    } else {
      if (rocblas_status st = chunk_logits(h, w, weight, E, d, c0, n, chunk); st != rocblas_status_success)
        return blas_error(fn, st);
      hipLaunchKernelGGL(chunk_grad_kernel, dim3(E), dim3(kRowThreads), 0, s, w.L, chunk, n, c0, edges->tgt, lse,
                         dloss, w.G);
    }
    // dhg^T [d, E] (+)= W_c^T [d, n] G_c^T [n, E]   (column-major views)
    rocblas_status st = gemm(h, rocblas_operation_none, rocblas_operation_none, d, E, n,
                             static_cast<const unsigned short*>(weight) + size_t(c0) * d, d, w.G, chunk,
                             c0 == 0 ? 0.f : 1.f, w.dhg, rocblas_datatype_f32_r, d);
    if (st != rocblas_status_success) return blas_error(fn, st);
    // dW_c^T [d, n] = hg^T [d, E] G_c [E, n]
    st = gemm(h, rocblas_operation_none, rocblas_operation_transpose, d, n, E, w.hg, d, w.G, chunk, 0.f,
              static_cast<unsigned short*>(dweight) + size_t(c0) * d, rocblas_datatype_bf16_r, d);
    if (st != rocblas_status_success) return blas_error(fn, st);
  }
  hipLaunchKernelGGL(scatter_rows_kernel, dim3(unsigned((int64_t(T) * pieces + 255) / 256)), dim3(256), 0, s, w.dhg,
                     edges->row_ptr, edges->ids, T, d, static_cast<uint4*>(dhidden));
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return hip_error(fn, e);
  return TREE_ATTN_OK;
}

}  // extern "C"
