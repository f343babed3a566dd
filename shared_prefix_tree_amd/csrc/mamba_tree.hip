// Mamba state forking on a shared-prefix forest: the tree-causal depthwise
// convolution and the scalar-decay state-space recurrence of a Mamba-2
// mixer, run along each token's ancestor path.
//
// The draft "feat(hybrid): add opt-in shared-prefix attention and Mamba
// execution" (intro) shares the prompt once, forks the recurrent state into
// each branch, runs the convolution halo per branch and accumulates the
// branches' gradients into the shared prefix; the issue "Shared-prefix
// training with context parallelism for exact agent trajectories" (section
// "Describe the solution you'd like") keeps convolution and recurrent state
// at branch points differentiable.  With prev(i) the token before i on its
// root-to-leaf path (the previous token of its segment, or the parent
// segment's last token for a segment's first token, none at a root):
//
//   conv:  y[i, c] = bias[c] + sum_{j < W} w[c, j] x[prev^(W-1-j)(i), c]
//   scan:  S_i = exp(dt[i,h] A[h]) S_prev(i) + dt[i,h] x[i,h,:] outer B[i,g,:]
//          y[i,h,:] = S_i C[i,g,:] + D[h] x[i,h,:]          (g = h / (H / G))
//
// Scan decomposition.  The plan cuts every segment into units of at most
// kUnit tokens; a unit's predecessor is the previous unit of its segment or
// the parent segment's last unit, so the units form a tree in DFS order.
// The state after a unit is linear in the state before it:
//   end(u) = decay(u) start(u) + local(u),  decay(u) = exp(A sum_{i in u} dt_i)
// 1. local:     per (unit, head), the unit from a zero state -> local(u),
//               decay(u)   (all units in parallel; 32 tokens at a time as one
//               rank-32 update of the state on the fp32 matrix cores);
// 2. propagate: per (head, quarter of the state), walk the units in DFS
//               order: start(u) = end(pred(u)); a fork reads its parent's
//               start and local back (each thread reads what it wrote);
// 3. output:    per (unit, head), scan again from start(u) and write y.
// The state before every 32-token chunk is kept for the backward pass.  In
// the output pass the state of one head (64 x N floats) is spread over a
// 256-thread block, two rows and N/8 columns per thread; y's sum over the
// state dimension is an eight-lane reduction.  Everything is fp32 with no
// atomics: results are bitwise reproducible.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <functional>
#include <memory>
#include <string>
#include <vector>

#include "../../include/tree_attn.h"
#include "mamba_plan.hpp"
#include "plan.hpp"

namespace tree_attn {
int report_error(int code, const std::string& msg);
int guard_host(const char* fn, const std::function<int()>& body) noexcept;
}

using tree_attn::report_error;

namespace {

constexpr int kUnit = tree_attn::kMambaUnit;  // tokens per scan unit
constexpr int kConvMaxWidth = tree_attn::kConvMaxWidth;
constexpr int kHalo = tree_attn::kConvHalo;
constexpr int kHeadDim = 64;       // P

}  // namespace

struct tree_attn_mamba_plan_s : tree_attn::MambaTables {
  int device = -1;  // -1: host-only plan
  void* block = nullptr;
  const int32_t *d_halo = nullptr, *d_csucc_ptr = nullptr, *d_csucc = nullptr;
  const int32_t *d_unit_start = nullptr, *d_unit_len = nullptr, *d_unit_pred = nullptr;
  const int32_t *d_usucc_ptr = nullptr, *d_usucc = nullptr, *d_uchain = nullptr;
};

namespace {

hipError_t upload_mamba_plan(tree_attn_mamba_plan_s& m) {
  const std::vector<int32_t>* parts[] = {&m.halo,     &m.csucc_ptr, &m.csucc,     &m.unit_start, &m.unit_len,
                                         &m.unit_pred, &m.usucc_ptr, &m.usucc,     &m.uchain};
  constexpr int kParts = 9;
  size_t off[kParts], total = 0;
  for (int k = 0; k < kParts; ++k) {
    off[k] = total;
    total += (parts[k]->size() * 4 + 255) & ~size_t(255);
  }
  std::vector<char> stage(std::max<size_t>(total, 256), 0);
  for (int k = 0; k < kParts; ++k)
    if (!parts[k]->empty()) std::memcpy(stage.data() + off[k], parts[k]->data(), parts[k]->size() * 4);
  hipError_t e = hipGetDevice(&m.device);
  if (e == hipSuccess) e = hipMalloc(&m.block, stage.size());
  if (e == hipSuccess) e = hipMemcpy(m.block, stage.data(), stage.size(), hipMemcpyHostToDevice);
  if (e != hipSuccess) return e;
  const int32_t** dst[] = {&m.d_halo,     &m.d_csucc_ptr, &m.d_csucc,      &m.d_unit_start, &m.d_unit_len,
                           &m.d_unit_pred, &m.d_usucc_ptr, &m.d_usucc, &m.d_uchain};
  for (int k = 0; k < kParts; ++k)
    *dst[k] = reinterpret_cast<const int32_t*>(static_cast<char*>(m.block) + off[k]);
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// convolution

// weights of channels c .. c+3 at tap j (w is [C][W])
template <int W>
__device__ inline void load_taps(const float* __restrict__ w, int c, float4 (&t)[W]) {
  if constexpr (W == 4) {
    const float4 r0 = reinterpret_cast<const float4*>(w + (c + 0) * 4)[0];
    const float4 r1 = reinterpret_cast<const float4*>(w + (c + 1) * 4)[0];
    const float4 r2 = reinterpret_cast<const float4*>(w + (c + 2) * 4)[0];
    const float4 r3 = reinterpret_cast<const float4*>(w + (c + 3) * 4)[0];
    t[0] = make_float4(r0.x, r1.x, r2.x, r3.x);
    t[1] = make_float4(r0.y, r1.y, r2.y, r3.y);
    t[2] = make_float4(r0.z, r1.z, r2.z, r3.z);
    t[3] = make_float4(r0.w, r1.w, r2.w, r3.w);
  } else {
#pragma unroll
    for (int j = 0; j < W; ++j) t[j] = make_float4(w[c * W + j], w[(c + 1) * W + j], w[(c + 2) * W + j], w[(c + 3) * W + j]);
  }
}

__device__ inline float4 fma4(float4 a, float4 b, float4 c) {
  return make_float4(fmaf(a.x, b.x, c.x), fmaf(a.y, b.y, c.y), fmaf(a.z, b.z, c.z), fmaf(a.w, b.w, c.w));
}

constexpr int kConvTokens = 16;  // tokens per block: the taps loaded once serve all of them

// one block per (16 tokens, 256 channel quads): a thread loads its taps once,
// issues the loads of all its 16 token rows together (the walk would otherwise
// have one row in flight at a time), and reads a tap k tokens back from those
// registers when it lies in the block's own rows on the same path (src = i - k);
// other sources (a segment's first tokens) are loaded when needed.  Halo
// indices are block-uniform.
template <int W>
__global__ __launch_bounds__(256) void conv_fwd_kernel(const float4* __restrict__ x, const float* __restrict__ w,
                                                       const float4* __restrict__ bias,
                                                       const int32_t* __restrict__ halo, int T, int C4,
                                                       float4* __restrict__ y) {
  const int c4 = blockIdx.y * blockDim.x + threadIdx.x;
  if (c4 >= C4) return;
  float4 t[W];
  load_taps<W>(w, 4 * c4, t);
  const float4 b = bias[c4];
  const int i0 = blockIdx.x * kConvTokens, n = min(T - i0, kConvTokens);
  float4 rows[kConvTokens];
#pragma unroll
  for (int q = 0; q < kConvTokens; ++q)
    rows[q] = q < n ? x[(size_t)(i0 + q) * C4 + c4] : make_float4(0.f, 0.f, 0.f, 0.f);
  // back[k - 1]: the row k tokens before the current one in the block (k <= kHalo)
  float4 back[kHalo];
#pragma unroll
  for (int k = 0; k < kHalo; ++k) back[k] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int q = 0; q < kConvTokens; ++q) {
    if (q < n) {
      const int i = i0 + q;
      float4 acc = fma4(t[W - 1], rows[q], b);
#pragma unroll
      for (int k = 1; k < W; ++k) {  // k steps back along the path: tap W-1-k (-1: the path is shorter)
        const int src = halo[(size_t)i * kHalo + k - 1];
        if (src >= 0) {
          float4 xs = back[k - 1];
          if (!(q >= k && src == i - k)) xs = x[(size_t)src * C4 + c4];
          acc = fma4(t[W - 1 - k], xs, acc);
        }
      }
      y[(size_t)i * C4 + c4] = acc;
    }
#pragma unroll
    for (int k = kHalo - 1; k > 0; --k) back[k] = back[k - 1];
    back[0] = rows[q];
  }
}

// dx[j] = w[:, W-1] dy[j] + sum over tokens i with prev^k(i) = j, 1 <= k < W,
// of w[:, W-1-k] dy[i]; every branch's halo lands on the shared prefix.  As in
// the forward, a thread issues the loads of its block's 16 dy rows together.
// A successor k tokens ahead on the same path (i = j + k, found in the halo
// table) is read from them when it lies in the block; the other successors (a
// branch point's children, listed in the successor table) and the rows past
// the block are loaded when needed.
template <int W>
__global__ __launch_bounds__(256) void conv_bwd_dx_kernel(const float4* __restrict__ dy, const float* __restrict__ w,
                                                          const int32_t* __restrict__ halo,
                                                          const int32_t* __restrict__ csucc_ptr,
                                                          const int32_t* __restrict__ csucc, int T, int C4,
                                                          float4* __restrict__ dx) {
  const int c4 = blockIdx.y * blockDim.x + threadIdx.x;
  if (c4 >= C4) return;
  float4 t[W];
  load_taps<W>(w, 4 * c4, t);
  const int j0 = blockIdx.x * kConvTokens, n = min(T - j0, kConvTokens);
  float4 rows[kConvTokens];
#pragma unroll
  for (int q = 0; q < kConvTokens; ++q)
    rows[q] = q < n ? dy[(size_t)(j0 + q) * C4 + c4] : make_float4(0.f, 0.f, 0.f, 0.f);
  // the other successors (a branch point's children), then the store
  auto dx_far = [&](int j, float4 acc) {
    for (int e = csucc_ptr[j]; e < csucc_ptr[j + 1]; ++e) {
      const int ent = csucc[e], i = ent >> 2, k = ent & 3;
      if (k >= W) continue;
      float4 tk = t[0];
#pragma unroll
      for (int r = 1; r < W; ++r)
        if (W - 1 - k == r) tk = t[r];
      acc = fma4(tk, dy[(size_t)i * C4 + c4], acc);
    }
    dx[(size_t)j * C4 + c4] = acc;
  };
  // the block's tokens in reverse, so that ahead[k - 1] holds the row k tokens ahead
  float4 ahead[kHalo];
#pragma unroll
  for (int k = 0; k < kHalo; ++k) ahead[k] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int q = kConvTokens - 1; q >= 0; --q) {
    if (q < n) {
      const int j = j0 + q;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      acc = fma4(t[W - 1], rows[q], acc);
#pragma unroll
      for (int k = 1; k < W; ++k) {  // the successor k tokens ahead, if j is its k-th predecessor
        const int i = j + k;
        if (i < T && halo[(size_t)i * kHalo + k - 1] == j) {
          float4 v = ahead[k - 1];
          if (q + k >= n) v = dy[(size_t)i * C4 + c4];  // past the block's rows
          acc = fma4(t[W - 1 - k], v, acc);
        }
      }
      dx_far(j, acc);
    }
#pragma unroll
    for (int k = kHalo - 1; k > 0; --k) ahead[k] = ahead[k - 1];
    ahead[0] = rows[q];
  }
}

constexpr int kConvRows = 256;  // tokens per partial of the weight gradient

// partial[b][c][k] = sum over tokens i of block b of dy[i, c] x[prev^k(i), c]
// for k < W, partial[b][c][kConvMaxWidth] = sum of dy[i, c]; one thread per
// four channels.  The thread walks its tokens in batches whose dy and x rows
// are loaded together, and keeps the x rows of the last kHalo tokens for the
// taps that reach back along the same path (prev^k(i) = i - k); other
// sources are loaded when needed.
constexpr int kDwBatch = 8;
__global__ void conv_bwd_dw_partial_kernel(const float4* __restrict__ x, const float4* __restrict__ dy,
                                           const int32_t* __restrict__ halo, int T, int C4, int W,
                                           float* __restrict__ partial) {
  const int c4 = blockIdx.y * blockDim.x + threadIdx.x;
  if (c4 >= C4) return;
  const int i0 = blockIdx.x * kConvRows, i1 = min(T, i0 + kConvRows);
  const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 acc[kConvMaxWidth + 1];
#pragma unroll
  for (int k = 0; k <= kConvMaxWidth; ++k) acc[k] = zero;
  float4 back[kHalo];  // back[k - 1]: the x row of the token k before the current one (in this walk)
#pragma unroll
  for (int k = 0; k < kHalo; ++k) back[k] = zero;
  for (int ib = i0; ib < i1; ib += kDwBatch) {
    float4 g[kDwBatch], xr[kDwBatch];
#pragma unroll
    for (int q = 0; q < kDwBatch; ++q) {
      const bool in = ib + q < i1;
      g[q] = in ? dy[(size_t)(ib + q) * C4 + c4] : zero;
      xr[q] = in ? x[(size_t)(ib + q) * C4 + c4] : zero;
    }
#pragma unroll
    for (int q = 0; q < kDwBatch; ++q) {
      const int i = ib + q;
      if (i < i1) {
        acc[kConvMaxWidth].x += g[q].x, acc[kConvMaxWidth].y += g[q].y, acc[kConvMaxWidth].z += g[q].z,
            acc[kConvMaxWidth].w += g[q].w;
        acc[0] = fma4(g[q], xr[q], acc[0]);
#pragma unroll
        for (int k = 1; k < kConvMaxWidth; ++k) {
          if (k < W) {
            const int src = halo[(size_t)i * kHalo + k - 1];
            if (src >= 0) {
              float4 xs = back[k - 1];
              if (!(src == i - k && i - k >= i0)) xs = x[(size_t)src * C4 + c4];
              acc[k] = fma4(g[q], xs, acc[k]);
            }
          }
        }
      }
#pragma unroll
      for (int k = kHalo - 1; k > 0; --k) back[k] = back[k - 1];
      back[0] = xr[q];
    }
  }
  float* out = partial + ((size_t)blockIdx.x * C4 * 4 + 4 * c4) * (kConvMaxWidth + 1);
#pragma unroll
  for (int k = 0; k <= kConvMaxWidth; ++k) {
    out[0 * (kConvMaxWidth + 1) + k] = acc[k].x;
    out[1 * (kConvMaxWidth + 1) + k] = acc[k].y;
    out[2 * (kConvMaxWidth + 1) + k] = acc[k].z;
    out[3 * (kConvMaxWidth + 1) + k] = acc[k].w;
  }
}

// dw[c][W-1-k] and dbias[c]: the partials summed in block order
__global__ void conv_bwd_dw_reduce_kernel(const float* __restrict__ partial, int nblk, int C, int W,
                                          float* __restrict__ dw, float* __restrict__ dbias) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= C) return;
  float acc[kConvMaxWidth + 1] = {};
  for (int b = 0; b < nblk; ++b) {
    const float* p = partial + ((long long)b * C + c) * (kConvMaxWidth + 1);
#pragma unroll
    for (int k = 0; k <= kConvMaxWidth; ++k) acc[k] += p[k];
  }
  for (int k = 0; k < W; ++k) dw[c * W + (W - 1 - k)] = acc[k];
  dbias[c] = acc[kConvMaxWidth];
}

// ---------------------------------------------------------------------------
// state-space scan

constexpr int kChunk = 32;                        // tokens staged in LDS at a time
constexpr int kChunksPerUnit = kUnit / kChunk;  // saved states per unit and head

struct ScanArgs {
  const float *x, *dt, *A, *B, *C, *D;
  const int32_t *unit_start, *unit_len, *unit_pred;
  int H, G, U;
  float* y;
  float* states;  // [U][kChunksPerUnit][H][P][N]: state before each chunk of each unit
  float* local;   // [U][H][P][N] unit scanned from a zero state
  float* decay;   // [U][H]
};

__host__ __device__ inline size_t state_index(int u, int chunk, int H, int h, int N) {
  return ((size_t(u) * kChunksPerUnit + chunk) * H + h) * size_t(kHeadDim) * N;
}

// ---------------------------------------------------------------------------
// fp32 matrix-core tiles
//
// In the chunk form of the recurrence every contraction over a chunk of 32
// tokens is a product of 32 x 32 tiles, run on the fp32 matrix cores
// (v_mfma_f32_32x32x2f32: lane l feeds A[l % 32][k0 + l / 32] and
// B[k0 + l / 32][l % 32]; accumulator r of lane l is
// C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]).  Operands are read from LDS
// with a per-lane address; the waves of a block share out the tiles by a
// fixed table, and a 64 x N state (or its gradient) stays in accumulator
// layout, one 32 x 32 tile per wave.
typedef float f32x16 __attribute__((ext_vector_type(16)));

// c += A B over K: A(i, k) = a[i AI + k AK], B(k, j) = b[k BK + j BJ].
// The contraction may run over k in any order, so the two halves of the
// wave take the two halves of k: consecutive products of a lane then read
// consecutive k, an operand that is contiguous in k (stride 1, 16-byte
// aligned rows) is read four products at a time with one 16-byte LDS read,
// and the next four products' operands are read while the current four run.
template <int S>
__device__ inline float4 read4(const float* p) {
  if constexpr (S == 1) {
    return *reinterpret_cast<const float4*>(p);
  } else {
    return make_float4(p[0], p[S], p[2 * S], p[3 * S]);
  }
}
template <int K, int AI, int AK, int BK, int BJ>
__device__ inline void mma_tile(f32x16& c, const float* a, const float* b, int ln) {
  static_assert(K % 8 == 0, "K in steps of 8");
  constexpr int KH = K / 2, NG = KH / 4;
  const int i = ln & 31, hk = ln >> 5;
  const float* pa = a + i * AI + hk * KH * AK;
  const float* pb = b + i * BJ + hk * KH * BK;
  float4 va = read4<AK>(pa), vb = read4<BK>(pb);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float4 na = va, nb = vb;
    if (g + 1 < NG) {
      na = read4<AK>(pa + 4 * (g + 1) * AK);
      nb = read4<BK>(pb + 4 * (g + 1) * BK);
    }
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(va.x, vb.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(va.y, vb.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(va.z, vb.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(va.w, vb.w, c, 0, 0, 0);
    va = na;
    vb = nb;
  }
}

// ln: the lane index, passed in so that a loop can make it opaque (address
// arithmetic is then redone per iteration instead of held in registers)
__device__ inline int tile_row(int r, int ln) { return 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3); }
__device__ inline int tile_col(int ln) { return ln & 31; }

// Cross-lane sums and scans with DPP lane moves, which stay in the vector
// unit (a shuffle goes through LDS and waits for it).  All lanes of the wave
// must be active.
template <int kCtrl, int kRowMask = 0xF>
__device__ inline float dpp(float v) {  // lanes whose source is invalid or masked get 0
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xF, false));
}
// sum over an aligned group of 8 lanes: pairs (quad_perm [1,0,3,2]), quads
// (quad_perm [2,3,0,1]), the other quad of the half-row (row_half_mirror);
// every lane of the group gets the same value
__device__ inline float sum8_dpp(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  return v;
}
// sum over an aligned group of 16 lanes (a DPP row): then the other half-row (row_mirror)
__device__ inline float sum16_dpp(float v) {
  v = sum8_dpp(v);
  v += dpp<0x140>(v);
  return v;
}
// inclusive scan over each aligned group of 32 lanes: within each 16-lane
// row by shifts of 1, 2, 4, 8 (row_shr), then the last lane of rows 0 and 2
// into every lane of rows 1 and 3 (row_bcast15 with row mask 0b1010)
__device__ inline float scan32_dpp(float v) {
  v += dpp<0x111>(v);
  v += dpp<0x112>(v);
  v += dpp<0x114>(v);
  v += dpp<0x118>(v);
  v += dpp<0x142, 0xA>(v);
  return v;
}
// the value of the lane below (wave_shr 1; lane 0 gets 0)
__device__ inline float lane_below_dpp(float v) { return dpp<0x138>(v); }

// l_k = sum_{j <= k} v_j over the 32 tokens of a chunk, v_j = dt_j A held by
// lane k of an aligned 32-lane group (an inclusive scan); all 64 lanes active
__device__ inline float chunk_log_decay(float v) {
  static_assert(kChunk == 32, "one chunk is one 32-lane scan");
  return scan32_dpp(v);
}

// barrier for LDS hand-offs only: global loads issued ahead stay in flight
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// fixed-order sum over the block (all threads get the result)
__device__ inline float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  lds_barrier();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  lds_barrier();
  float r = 0.f;
  for (int w = 0; w < int(blockDim.x) / 64; ++w) r += red[w];
  return r;
}

constexpr int kFwdThreads = 512;
constexpr int kFX = kHeadDim + 4;  // x rows in LDS (16-byte aligned, banks staggered)

template <int N>
struct FwdSmem {
  static constexpr int PB = N + 4;
  float x[kChunk * kFX], xw[kChunk * kFX];  // x rows; x_j scaled by w_j
  float B[kChunk * PB];
  float dt[kChunk], l[kChunk], w[kChunk];   // w_j = e^(l_e - l_j) dt_j
};

// Unit-local passes in chunk form: one block of eight waves per (unit,
// head); wave w owns 32 x 32 tile w of a 64 x N accumulator.  Per chunk of
// 32 tokens, with l_i = A times the sum of dt over the chunk up to and
// including token i, and l_b that sum over the unit's earlier chunks:
//   forward (kGrad = false): S <- e^(l_e) S + sum_j (e^(l_e - l_j) dt_j x_j) outer B_j
//       from a zero state: S = local(u);
//   backward (kGrad = true): L <- L + sum_k (e^(l_b + l_k) dy_k) outer C_k
//       = local_in(u), the gradient reaching the unit's start from inside.
// Both are one rank-32 tile product per chunk on the fp32 matrix cores.
// decay(u) = e^(A sum dt) either way.
struct LocalArgs {
  const float *v, *w, *dt, *A;  // v: x or dy [T][H][64]; w: B or C [T][G][N]
  const int32_t *unit_start, *unit_len;
  int H, G;
  float* out;    // [U][H][64][N]
  float* decay;  // [U][H]
};

template <int N, bool kGrad>
__global__ __launch_bounds__(kFwdThreads) void ssm_unit_local_kernel(LocalArgs a) {
  constexpr int PB = FwdSmem<N>::PB, NT = N / 32, GT = 2 * NT;
  __shared__ __attribute__((aligned(16))) FwdSmem<N> sm;
  const int u = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int g = h / (a.H / a.G);
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = a.unit_start[u], len = a.unit_len[u];
  const float Ah = a.A[h];
  const bool sown = wave < GT;
  const int sp = wave / NT, sn = wave % NT;  // tile: rows 32 sp .., columns 32 sn ..
  f32x16 S = f32x16{};
  float lsum = 0.f;
  for (int ci = 0; ci * kChunk < len; ++ci) {
    const int c0 = t0 + ci * kChunk, clen = min(kChunk, len - ci * kChunk);
    int ln = tid & 63;
    asm volatile("" : "+v"(ln));
    // stage the chunk (padding: zeros)
    for (int e = tid; e < kChunk * (kHeadDim / 4); e += kFwdThreads) {
      const int k = e / (kHeadDim / 4), q = e % (kHeadDim / 4);
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (k < clen) v = reinterpret_cast<const float4*>(a.v + ((size_t)(c0 + k) * a.H + h) * kHeadDim)[q];
      *reinterpret_cast<float4*>(&sm.x[k * kFX + 4 * q]) = v;
    }
    for (int e = tid; e < kChunk * (N / 4); e += kFwdThreads) {
      const int k = e / (N / 4), q = e % (N / 4);
      float4 vb = make_float4(0.f, 0.f, 0.f, 0.f);
      if (k < clen) vb = reinterpret_cast<const float4*>(a.w + ((size_t)(c0 + k) * a.G + g) * N)[q];
      *reinterpret_cast<float4*>(&sm.B[k * PB + 4 * q]) = vb;
    }
    if (tid < kChunk) sm.dt[tid] = tid < clen ? a.dt[(size_t)(c0 + tid) * a.H + h] : 0.f;
    lds_barrier();
    if (tid < 64) {  // l_k = sum_{j <= k} dt_j A: a scan over the 32 lanes of a half-wave
      const int k = tid & (kChunk - 1);
      const float l = chunk_log_decay(sm.dt[k] * Ah);
      const float le = __shfl(l, kChunk - 1, kChunk);
      if (tid < kChunk) {
        sm.l[k] = l;
        sm.w[k] = kGrad ? __expf(lsum + l) : __expf(le - l) * sm.dt[k];
      }
    }
    lds_barrier();
    const float le = sm.l[kChunk - 1];
    lsum += le;
    for (int e = tid; e < kChunk * (kHeadDim / 4); e += kFwdThreads) {
      const int j = e / (kHeadDim / 4), q = e % (kHeadDim / 4);
      const float wj = sm.w[j];
      float4 v = *reinterpret_cast<const float4*>(&sm.x[j * kFX + 4 * q]);
      v.x *= wj, v.y *= wj, v.z *= wj, v.w *= wj;
      *reinterpret_cast<float4*>(&sm.xw[j * kFX + 4 * q]) = v;
    }
    lds_barrier();
    if (sown) {
      if (!kGrad) {
        const float ele = __expf(le);
#pragma unroll
        for (int r = 0; r < 16; ++r) S[r] *= ele;
      }
      mma_tile<kChunk, 1, kFX, PB, 1>(S, sm.xw + 32 * sp, sm.B + 32 * sn, ln);
    }
    lds_barrier();
  }
  if (sown) {
    const size_t base = (size_t(u) * a.H + h) * kHeadDim * N;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      a.out[base + size_t(32 * sp + tile_row(r, tid & 63)) * N + 32 * sn + tile_col(tid & 63)] = S[r];
  }
  if (tid == 0) a.decay[(size_t)u * a.H + h] = __expf(lsum);
}

constexpr float kRefStep = 32.f;  // log-space step of the output pass's state reference

// output pass: one block per (unit, head) from the unit's start state;
// thread (row pair pr, column group ng) holds rows 2 pr, 2 pr + 1 x columns
// [ng NC, (ng+1) NC); y's sum over columns is an eight-lane reduction.  The
// state before every chunk after the first is saved for the backward pass.
template <int N>
__global__ __launch_bounds__(256) void ssm_output_kernel(ScanArgs a) {
  constexpr int NG = 8, NC = N / NG;
  __shared__ __attribute__((aligned(16))) float sB[kChunk][N];
  __shared__ __attribute__((aligned(16))) float sC[kChunk][N];
  __shared__ __attribute__((aligned(16))) float sX[kChunk][kHeadDim];
  __shared__ float sDF[kChunk], sG[kChunk], sRho[kChunk];
  const int u = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int g = h / (a.H / a.G);
  const int tid = threadIdx.x, ng = tid & (NG - 1), pr = tid / NG;
  const int t0 = a.unit_start[u], len = a.unit_len[u];
  const float Ah = a.A[h], Dh = a.D[h];
  float S[2][NC];
  {
    const float* s0 = a.states + state_index(u, 0, a.H, h, N) + size_t(2 * pr) * N + ng * NC;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int m = 0; m < NC / 4; ++m) {
        const float4 v = reinterpret_cast<const float4*>(s0 + r * N)[m];
        S[r][4 * m] = v.x, S[r][4 * m + 1] = v.y, S[r][4 * m + 2] = v.z, S[r][4 * m + 3] = v.w;
      }
  }
  for (int ci = 0; ci * kChunk < len; ++ci) {
    const int c0 = t0 + ci * kChunk, clen = min(kChunk, len - ci * kChunk);
    if (ci > 0) {
      float* sv = a.states + state_index(u, ci, a.H, h, N) + size_t(2 * pr) * N + ng * NC;
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int m = 0; m < NC / 4; ++m)
          reinterpret_cast<float4*>(sv + r * N)[m] =
              make_float4(S[r][4 * m], S[r][4 * m + 1], S[r][4 * m + 2], S[r][4 * m + 3]);
    }
    __syncthreads();
    for (int e = tid; e < kChunk * (N / 4); e += 256) {
      const int k = e / (N / 4), q = e % (N / 4);
      const size_t off = ((size_t)(c0 + k) * a.G + g) * N;
      float4 vb = make_float4(0.f, 0.f, 0.f, 0.f), vc = vb;
      if (k < clen) {
        vb = reinterpret_cast<const float4*>(a.B + off)[q];
        vc = reinterpret_cast<const float4*>(a.C + off)[q];
      }
      reinterpret_cast<float4*>(sB[k])[q] = vb;
      reinterpret_cast<float4*>(sC[k])[q] = vc;
    }
    for (int e = tid; e < kChunk * (kHeadDim / 4); e += 256) {
      const int k = e / (kHeadDim / 4), q = e % (kHeadDim / 4);
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (k < clen) v = reinterpret_cast<const float4*>(a.x + ((size_t)(c0 + k) * a.H + h) * kHeadDim)[q];
      reinterpret_cast<float4*>(sX[k])[q] = v;
    }
    // The state is kept as S~ = e^(R - l_k) S against a reference R that is
    // a multiple of kRefStep in log space (R_k = kRefStep ceil(l_k / kRefStep),
    // so 1 <= e^(R - l_k) < e^kRefStep): a token's update is then one fma per
    // element, S~ += e^(R - l_k) dt_k x_k B_k, and y_k = e^(l_k - R) S~ C_k.
    // When R moves, S~ is rescaled by e^(R_new - R_old).  Per token: sDF =
    // dt e^(R - l), sG = e^(l - R), sRho = the rescale (1: none).
    if (tid < 64) {
      const int k = tid & (kChunk - 1);
      const float d = k < clen ? a.dt[(size_t)(c0 + k) * a.H + h] : 0.f;
      const float l = chunk_log_decay(d * Ah);
      const float ref = kRefStep * ceilf(l * (1.f / kRefStep));
      float prev = __shfl_up(ref, 1, kChunk);
      if (k == 0) prev = 0.f;
      if (tid < kChunk) {
        sDF[k] = d * expf(ref - l);
        sG[k] = expf(l - ref);
        sRho[k] = ref == prev ? 1.f : expf(ref - prev);
      }
    }
    __syncthreads();
    for (int k = 0; k < clen; ++k) {
      const float df = sDF[k], gk = sG[k], rho = sRho[k];
      if (rho != 1.f) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int m = 0; m < NC; ++m) S[r][m] *= rho;
      }
      const float x0 = sX[k][2 * pr], x1 = sX[k][2 * pr + 1];
      const float u0 = df * x0, u1 = df * x1;
      float y0 = 0.f, y1 = 0.f;
#pragma unroll
      for (int m = 0; m < NC / 4; ++m) {
        const float4 b = reinterpret_cast<const float4*>(&sB[k][ng * NC])[m];
        const float4 c = reinterpret_cast<const float4*>(&sC[k][ng * NC])[m];
#define TREE_SSM_STEP(J, BJ, CJ)                                   \
  S[0][4 * m + J] = fmaf(u0, BJ, S[0][4 * m + J]);                 \
  S[1][4 * m + J] = fmaf(u1, BJ, S[1][4 * m + J]);                 \
  y0 = fmaf(S[0][4 * m + J], CJ, y0);                              \
  y1 = fmaf(S[1][4 * m + J], CJ, y1);
        TREE_SSM_STEP(0, b.x, c.x)
        TREE_SSM_STEP(1, b.y, c.y)
        TREE_SSM_STEP(2, b.z, c.z)
        TREE_SSM_STEP(3, b.w, c.w)
#undef TREE_SSM_STEP
      }
      y0 = sum8_dpp(y0);
      y1 = sum8_dpp(y1);
      if (ng == 0)
        *reinterpret_cast<float2*>(a.y + ((size_t)(c0 + k) * a.H + h) * kHeadDim + 2 * pr) =
            make_float2(fmaf(Dh, x0, gk * y0), fmaf(Dh, x1, gk * y1));
    }
    {  // back to the state itself at the chunk's end
      const float ge = sG[clen - 1];
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int m = 0; m < NC; ++m) S[r][m] *= ge;
    }
  }
}

constexpr int kWalkAhead = 8;   // units whose state rows are in flight ahead of the walk
constexpr int kWalkTile = 256;  // walk steps whose unit tables are staged in LDS at a time

template <int NE>
__device__ inline void load_row_part(const float* p, float (&v)[NE]) {
  static_assert(NE % 4 == 0, "whole float4 pieces");
#pragma unroll
  for (int m = 0; m < NE / 4; ++m) {
    const float4 t = reinterpret_cast<const float4*>(p)[m];
    v[4 * m] = t.x, v[4 * m + 1] = t.y, v[4 * m + 2] = t.z, v[4 * m + 3] = t.w;
  }
}

template <int NE>
__device__ inline void store_row_part(float* p, const float (&v)[NE]) {
#pragma unroll
  for (int m = 0; m < NE / 4; ++m)
    reinterpret_cast<float4*>(p)[m] = make_float4(v[4 * m], v[4 * m + 1], v[4 * m + 2], v[4 * m + 3]);
}

// one block per (head, quarter of the rows); thread holds row p, columns
// [c NE2, (c+1) NE2); walks the units in DFS order.  The walk's unit tables
// (predecessor, decay) are staged in LDS a tile at a time, and each unit's
// local row, which does not depend on the walk, is loaded kWalkAhead units
// ahead into a register ring; the loop is unrolled over the ring so every
// slot index is a constant.
template <int N>
__global__ __launch_bounds__(256) void ssm_propagate_kernel(ScanArgs a) {
  constexpr int NE2 = N / 16, R = kWalkAhead;
  __shared__ int sPred[kWalkTile];
  __shared__ float sDec[kWalkTile];
  const int h = blockIdx.x >> 2, quarter = blockIdx.x & 3;
  const int p = quarter * 16 + (threadIdx.x >> 4), c = threadIdx.x & 15;
  const size_t col = size_t(p) * N + c * NE2;
  const size_t lstride = size_t(a.H) * kHeadDim * N;
  const size_t loff = size_t(h) * kHeadDim * N + col;
  float rloc[R][NE2];
  auto load = [&](int u, int slot) {
    if (u < a.U) load_row_part<NE2>(a.local + u * lstride + loff, rloc[slot]);
  };
#pragma unroll
  for (int j = 0; j < R; ++j) load(j, j);
  float end[NE2];
#pragma unroll
  for (int k = 0; k < NE2; ++k) end[k] = 0.f;
  for (int base = 0; base < a.U; base += R) {
    if (base % kWalkTile == 0) {
      __syncthreads();
      for (int t = threadIdx.x; t < kWalkTile && base + t < a.U; t += blockDim.x) {
        sPred[t] = a.unit_pred[base + t];
        sDec[t] = a.decay[(size_t)(base + t) * a.H + h];
      }
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int u = base + j;
      if (u >= a.U) break;
      const int pred = sPred[u % kWalkTile];
      float start[NE2];
      if (pred < 0) {
#pragma unroll
        for (int k = 0; k < NE2; ++k) start[k] = 0.f;
      } else if (pred == u - 1) {
#pragma unroll
        for (int k = 0; k < NE2; ++k) start[k] = end[k];
      } else {  // a fork: the parent's end, from what this thread stored
        const float dp = a.decay[(size_t)pred * a.H + h];
        float sp[NE2], lp[NE2];
        load_row_part<NE2>(a.states + state_index(pred, 0, a.H, h, N) + col, sp);
        load_row_part<NE2>(a.local + pred * lstride + loff, lp);
#pragma unroll
        for (int k = 0; k < NE2; ++k) start[k] = fmaf(dp, sp[k], lp[k]);
      }
      store_row_part<NE2>(a.states + state_index(u, 0, a.H, h, N) + col, start);
      const float du = sDec[u % kWalkTile];
#pragma unroll
      for (int k = 0; k < NE2; ++k) end[k] = fmaf(du, start[k], rloc[j][k]);
      load(u + R, j);
    }
  }
}

template <int N>
hipError_t launch_ssm_fwd(const ScanArgs& a, hipStream_t s) {
  const dim3 grid(unsigned(a.U) * unsigned(a.H));
  const LocalArgs la{a.x, a.B, a.dt, a.A, a.unit_start, a.unit_len, a.H, a.G, a.local, a.decay};
  hipLaunchKernelGGL((ssm_unit_local_kernel<N, false>), grid, dim3(kFwdThreads), 0, s, la);
  hipLaunchKernelGGL((ssm_propagate_kernel<N>), dim3(unsigned(a.H) * 4), dim3(256), 0, s, a);
  hipLaunchKernelGGL((ssm_output_kernel<N>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// state-space backward
//
// dS_i, the gradient of the loss with respect to S_i, obeys
//   dS_i = dy_i outer C_i + sum over successors k of i of a_k dS_k,
// so at a branch point the branches' gradients add up.  Per unit the
// gradient reaching the state before it is linear in the gradient leaving
// its last token:  in(u) = local_in(u) + decay(u) out(u),
//   local_in(u) = sum_{k in u} exp(l_k) dy_k outer C_k   (l_k: A times the
//   sum of dt over the unit's tokens up to and including k),
//   out(u)      = sum over successor units v of in(v).
// 4. local_in:   per (unit, head), local_in(u) and decay(u);
// 5. propagate:  per (head, quarter), walk the units in reverse DFS order;
// 6. gradients:  per (unit, head), the unit in chunks of 32 tokens, last
//    chunk first, in the chunk (dual) form of the recurrence: with S0 the
//    state before the chunk and G the gradient leaving its last token,
//      S_i  = exp(l_i) S0 + sum_{j<=i} exp(l_i - l_j) dt_j x_j outer B_j
//      dS_i = sum_{k>=i} exp(l_k - l_i) dy_k outer C_k + exp(l_e - l_i) G
//    (l now cumulative over the chunk, l_e its last value), which gives
//      dx_i = D dy_i + dt_i [sum_{k>=i} e^(l_k-l_i) (C_k.B_i) dy_k + e^(l_e-l_i) G B_i]
//      dB_i = dt_i [sum_{k>=i} e^(l_k-l_i) (x_i.dy_k) C_k + e^(l_e-l_i) G^T x_i]
//      dC_k = e^(l_k) S0^T dy_k + sum_{j<=k} e^(l_k-l_j) dt_j (x_j.dy_k) B_j
//      a_i <dS_i, S_{i-1}> = sum_{k>=i} e^(l_k) (S0^T dy_k).C_k
//          + sum_{k>=i} sum_{j<i} e^(l_k-l_j) dt_j (x_j.dy_k)(C_k.B_j)
//          + e^(l_e) <G, S0> + sum_{j<i} e^(l_e-l_j) dt_j x_j.(G B_j)
//      ddt_i = x_i.(dS_i B_i) + A a_i <dS_i, S_{i-1}>,  dA = sum_i dt_i a_i <dS_i, S_{i-1}>
//    Every exponent is <= 0.  The chunk's start states come from one
//    forward sweep over the unit from the saved start(u); G from out(u),
//    moved back one chunk at a time.  dB and dC are summed over the heads
//    of a group (in place over the heads a block takes in turn, then over
//    those blocks), and dA, dD over units, all in fixed orders.

struct ScanBwdArgs {
  const float *x, *dt, *A, *B, *C, *D, *dy, *states;
  const int32_t *unit_start, *unit_len, *unit_pred, *usucc_ptr, *usucc, *uchain;
  int H, G, U, T;
  float* in;      // [U][H][P][N]: local_in, then in(u)
  float* gout;    // [U][H][P][N]: out(u)
  float* decay;   // [U][H]
  int hpb;        // heads per block of the gradient pass (they share a group)
  float* dB_part; // [T][H / hpb][N]: per block of heads
  float* dC_part; // [T][H / hpb][N]
  float* dA_part; // [U][H]
  float* dD_part; // [U][H]
  float *dx, *ddt, *dA, *dB, *dC, *dD;
};

// reverse DFS walk, staged like the forward walk
template <int N>
__global__ __launch_bounds__(256) void ssm_bwd_propagate_kernel(ScanBwdArgs a) {
  constexpr int NE2 = N / 16, R = kWalkAhead;
  __shared__ int sChain[kWalkTile];
  __shared__ float sDec[kWalkTile];
  const int h = blockIdx.x >> 2, quarter = blockIdx.x & 3;
  const int p = quarter * 16 + (threadIdx.x >> 4), c = threadIdx.x & 15;
  const size_t ustride = size_t(a.H) * kHeadDim * N;
  const size_t hoff = size_t(h) * kHeadDim * N + size_t(p) * N + c * NE2;
  float rin[R][NE2];
  // walk step t visits unit U - 1 - t
  auto load = [&](int t, int slot) {
    if (t < a.U) load_row_part<NE2>(a.in + size_t(a.U - 1 - t) * ustride + hoff, rin[slot]);
  };
#pragma unroll
  for (int j = 0; j < R; ++j) load(j, j);
  float next_in[NE2];  // in(u + 1)
#pragma unroll
  for (int k = 0; k < NE2; ++k) next_in[k] = 0.f;
  for (int base = 0; base < a.U; base += R) {
    if (base % kWalkTile == 0) {
      __syncthreads();
      for (int t = threadIdx.x; t < kWalkTile && base + t < a.U; t += blockDim.x) {
        const int u = a.U - 1 - (base + t);
        sChain[t] = a.uchain[u];
        sDec[t] = a.decay[(size_t)u * a.H + h];
      }
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int t = base + j;
      if (t >= a.U) break;
      const int u = a.U - 1 - t;
      float G[NE2];
      if (sChain[t % kWalkTile]) {
#pragma unroll
        for (int k = 0; k < NE2; ++k) G[k] = next_in[k];
      } else {  // a branch point (or a leaf): the successors' in(v), ascending
#pragma unroll
        for (int k = 0; k < NE2; ++k) G[k] = 0.f;
        for (int e = a.usucc_ptr[u]; e < a.usucc_ptr[u + 1]; ++e) {
          float iv[NE2];
          load_row_part<NE2>(a.in + size_t(a.usucc[e]) * ustride + hoff, iv);
#pragma unroll
          for (int k = 0; k < NE2; ++k) G[k] += iv[k];
        }
      }
      const float du = sDec[t % kWalkTile];
#pragma unroll
      for (int k = 0; k < NE2; ++k) next_in[k] = fmaf(du, G[k], rin[j][k]);
      store_row_part<NE2>(a.gout + size_t(u) * ustride + hoff, G);
      store_row_part<NE2>(a.in + size_t(u) * ustride + hoff, next_in);
      load(t + R, j);
    }
  }
}

constexpr int kBwdThreads = 512;

constexpr int kPX = kHeadDim + 4;  // x, dy, (G B_j) and bracket rows (16-byte aligned rows)
constexpr int kPZ = kChunk + 1;    // 32 x 32 matrices read along rows and columns
constexpr int kPW = kChunk + 4;    // 32 x 32 matrices read as matrix-core operands (16-byte rows)

template <int N>
struct BwdSmem {
  static constexpr int PB = N + 4;  // B, C, S0, G rows
  float x[kChunk * kPX], dy[kChunk * kPX];
  float B[kChunk * PB], C[kChunk * PB];
  float S0[kHeadDim * PB], G[kHeadDim * PB];  // reused as S0^T dy and G^T x ([k][n]) after the first products
  float CB[kChunk * kPZ], XD[kChunk * kPZ];   // [k][j]: C_k.B_j, x_j.dy_k
  float Z[kChunk * kPZ];                      // [k][i]: sum over j < min(i, k) of e^(l_k-l_j) dt_j XD CB
  float W1[kChunk * kPW], W2[kChunk * kPW], W3[kChunk * kPW];
  float GB[kChunk * kPX];                     // [j][p]: (G B_j)[p], then the dx bracket
  float dt[kChunk], l[kChunk], q[kChunk], r[kChunk], s[kChunk];
  float red[kBwdThreads / 64];
};

// first products of a chunk, shared out over the waves:
//   0: C B^T, 1: X D, 2..: G B (per 32 rows of G), then S0^T dy and G^T x (per 32 columns)
template <int N>
struct FirstJobs {
  static constexpr int NT = N / 32;
  // job ids per wave (-1: none); N = 128: CB | GB0 | GB1 | XD, S0dy0 | S0dy1, S0dy2 | S0dy3, Gx0 | Gx1, Gx2 | Gx3
  static __device__ inline int job(int w, int slot) {
    if constexpr (N == 128) {
      if (slot == 0) return w == 0 ? 0 : w == 1 ? 2 : w == 2 ? 3 : w == 3 ? 1 : 2 * w - 3;
      return w == 3 ? 4 : (w >= 4 && w <= 6) ? 2 * w - 2 : -1;
    } else {
      if (slot == 1) return -1;
      return w == 0 ? 0 : w == 1 ? 2 : w == 2 ? 3 : w == 3 ? 1 : w;
    }
  }
};

template <int N>
__device__ __forceinline__ void ssm_bwd_grad_head(const ScanBwdArgs& a, BwdSmem<N>& sm, int u, int h, int hp,
                                                  int hh) {
  constexpr int PB = BwdSmem<N>::PB;
  constexpr int NT = N / 32;            // 32-column tiles of the state
  constexpr int GT = 2 * NT;            // 32 x 32 tiles of the 64 x N state
  const int HP = a.H / a.hpb;           // blocks of heads
  const int g = h / (a.H / a.G);
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = a.unit_start[u], len = a.unit_len[u];
  const int nch = (len + kChunk - 1) / kChunk;
  const float Ah = a.A[h], Dh = a.D[h];
  const size_t hrow = (size_t(u) * a.H + h) * kHeadDim * N;

  // this wave's tile of G (and of S0): rows 32 gp .., columns 32 gn ..
  const bool gown = wave < GT;
  const int gp = wave / NT, gn = wave % NT;
  f32x16 Gt;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    Gt[r] = gown ? a.gout[hrow + size_t(32 * gp + tile_row(r, tid & 63)) * N + 32 * gn + tile_col(tid & 63)] : 0.f;
  float dA_acc = 0.f, dD_acc = 0.f;

  // the next chunk's inputs are loaded into registers while this one is
  // processed (x, dy: one float4 per thread; B, C: N / 64 each)
  constexpr int NBC = N / 64;
  float4 pfx, pfy, pfb[NBC], pfc[NBC];
  float pfdt = 0.f, pfs[16];
  auto fetch = [&](int c) {
    const int c0 = t0 + c * kChunk, clen = min(kChunk, len - c * kChunk);
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    {
      const int k = tid / (kHeadDim / 4), q = tid % (kHeadDim / 4);
      pfx = pfy = z;
      if (k < clen) {
        const size_t off = ((size_t)(c0 + k) * a.H + h) * kHeadDim;
        pfx = reinterpret_cast<const float4*>(a.x + off)[q];
        pfy = reinterpret_cast<const float4*>(a.dy + off)[q];
      }
    }
#pragma unroll
    for (int m = 0; m < NBC; ++m) {
      const int e = tid + m * kBwdThreads, k = e / (N / 4), q = e % (N / 4);
      pfb[m] = pfc[m] = z;
      if (k < clen) {
        const size_t off = ((size_t)(c0 + k) * a.G + g) * N;
        pfb[m] = reinterpret_cast<const float4*>(a.B + off)[q];
        pfc[m] = reinterpret_cast<const float4*>(a.C + off)[q];
      }
    }
    pfdt = tid < clen ? a.dt[(size_t)(c0 + tid) * a.H + h] : 0.f;
    if (gown) {
      const float* s0 = a.states + state_index(u, c, a.H, h, N);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        pfs[r] = s0[size_t(32 * gp + tile_row(r, tid & 63)) * N + 32 * gn + tile_col(tid & 63)];
    }
  };
  fetch(nch - 1);

  for (int c = nch - 1; c >= 0; --c) {
    const int c0 = t0 + c * kChunk, clen = min(kChunk, len - c * kChunk);
    int ln = tid & 63;
    asm volatile("" : "+v"(ln));
    // stage the chunk (padding: zeros, so padded tokens contribute nothing)
    {
      const int k = tid / (kHeadDim / 4), q = tid % (kHeadDim / 4);
      *reinterpret_cast<float4*>(&sm.x[k * kPX + 4 * q]) = pfx;
      *reinterpret_cast<float4*>(&sm.dy[k * kPX + 4 * q]) = pfy;
    }
#pragma unroll
    for (int m = 0; m < NBC; ++m) {
      const int e = tid + m * kBwdThreads, k = e / (N / 4), q = e % (N / 4);
      *reinterpret_cast<float4*>(&sm.B[k * PB + 4 * q]) = pfb[m];
      *reinterpret_cast<float4*>(&sm.C[k * PB + 4 * q]) = pfc[m];
    }
    if (tid < kChunk) sm.dt[tid] = pfdt;
    // the state before the chunk (saved by the forward) and G, into LDS; <G, S0>
    float gs = 0.f;
    if (gown) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * gp + tile_row(r, ln), col = 32 * gn + tile_col(ln);
        sm.S0[row * PB + col] = pfs[r];
        sm.G[row * PB + col] = Gt[r];
        gs = fmaf(Gt[r], pfs[r], gs);
      }
    }
    // this lane's dB / dC entries of the chunk from the block's earlier heads,
    // read before the next chunk's inputs (loads complete in order, so using
    // them then does not wait for those)
    float prevC[16], prevB[16];
    if (hh > 0 && wave < NT) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int k = tile_row(r, ln);
        const size_t e = ((size_t)(c0 + min(k, clen - 1)) * HP + hp) * N + 32 * wave + tile_col(ln);
        prevC[r] = a.dC_part[e];
        prevB[r] = a.dB_part[e];
      }
    }
    if (c > 0) fetch(c - 1);  // in flight during this chunk
    lds_barrier();
    if (tid < 64) {  // the scan runs on a whole wave (lanes 32.. repeat it)
      const int k = tid & (kChunk - 1);
      const float l = chunk_log_decay(sm.dt[k] * Ah);
      if (tid < kChunk) sm.l[k] = l;
    }
    gs = block_sum(gs, sm.red);  // (its barriers also publish l)

    // first products
    f32x16 acc[2];
    int jobs[2];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      jobs[sl] = FirstJobs<N>::job(wave, sl);
      acc[sl] = f32x16{};
      const int j = jobs[sl];
      if (j == 0) {
        mma_tile<N, PB, 1, 1, PB>(acc[sl], sm.C, sm.B, ln);  // CB(k, j) = C_k . B_j
      } else if (j == 1) {
        mma_tile<kHeadDim, kPX, 1, 1, kPX>(acc[sl], sm.dy, sm.x, ln);  // XD(k, j) = dy_k . x_j
      } else if (j >= 2 && j < 4) {
        const int pt = j - 2;  // GB(j, p) = B_j . G_p, rows p in 32 pt ..
        mma_tile<N, PB, 1, 1, PB>(acc[sl], sm.B, sm.G + 32 * pt * PB, ln);
      } else if (j >= 4 && j < 4 + NT) {
        const int nt = j - 4;  // S0^T dy: (k, n) = sum_p dy[k][p] S0[p][n]
        mma_tile<kHeadDim, kPX, 1, PB, 1>(acc[sl], sm.dy, sm.S0 + 32 * nt, ln);
      } else if (j >= 4 + NT) {
        const int nt = j - 4 - NT;  // G^T x: (k, n) = sum_p x[k][p] G[p][n]
        mma_tile<kHeadDim, kPX, 1, PB, 1>(acc[sl], sm.x, sm.G + 32 * nt, ln);
      }
    }
    lds_barrier();  // S0 and G are overwritten below
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int j = jobs[sl];
      if (j < 0) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = tile_row(r, ln), col = tile_col(ln);
        if (j == 0) sm.CB[row * kPZ + col] = acc[sl][r];
        else if (j == 1) sm.XD[row * kPZ + col] = acc[sl][r];
        else if (j < 4) sm.GB[row * kPX + 32 * (j - 2) + col] = acc[sl][r];
        else if (j < 4 + NT) sm.S0[row * PB + 32 * (j - 4) + col] = acc[sl][r];
        else sm.G[row * PB + 32 * (j - 4 - NT) + col] = acc[sl][r];
      }
    }
    lds_barrier();
    const float le = sm.l[kChunk - 1];
    const float ele = __expf(le);
    // decay-weighted 32 x 32 matrices
    for (int e = tid; e < kChunk * kChunk; e += kBwdThreads) {
      const int k = e / kChunk, j = e % kChunk;
      const float lk = sm.l[k], lj = sm.l[j];
      const float xd = sm.XD[k * kPZ + j];
      sm.W1[k * kPW + j] = j <= k ? __expf(lk - lj) * sm.dt[j] * xd : 0.f;              // dC: sources j <= k
      sm.W2[k * kPW + j] = j >= k ? __expf(lj - lk) * sm.XD[j * kPZ + k] : 0.f;         // dB: readers j >= k
      sm.W3[k * kPW + j] = j >= k ? __expf(lj - lk) * sm.CB[j * kPZ + k] : 0.f;         // dx: readers j >= k
      // Z(k, i) = sum_{j < i} e^(l_k-l_j) dt_j XD CB over j < k: an exclusive scan along the row,
      // whose 32 entries are the 32 lanes of a half-wave (every lane takes part: 1024 = 2 x 512)
      const float z = j < k ? __expf(lk - lj) * sm.dt[j] * xd * sm.CB[k * kPZ + j] : 0.f;
      const float zx = scan32_dpp(z);  // inclusive; the exclusive value is the lane below's
      const float zb = lane_below_dpp(zx);
      sm.Z[k * kPZ + j] = j > 0 ? zb : 0.f;
    }
    // per-token sums: q_k = e^(l_k) (S0^T dy_k).C_k, r'_j = e^(l_e-l_j) dt_j x_j.(G B_j), dD
    {
      const int k = tid >> 4, sub = tid & 15;  // 16 lanes per token
      float qv = 0.f, rv = 0.f, dd = 0.f;
      for (int n = sub; n < N; n += 16) qv = fmaf(sm.S0[k * PB + n], sm.C[k * PB + n], qv);
      for (int p = sub; p < kHeadDim; p += 16) {
        rv = fmaf(sm.x[k * kPX + p], sm.GB[k * kPX + p], rv);
        dd = fmaf(sm.x[k * kPX + p], sm.dy[k * kPX + p], dd);
      }
      qv = sum16_dpp(qv);
      rv = sum16_dpp(rv);
      dd = sum16_dpp(dd);
      if (sub == 0) {
        const float lk = sm.l[k];
        sm.q[k] = __expf(lk) * qv;
        sm.r[k] = __expf(le - lk) * sm.dt[k] * rv;
        dD_acc += dd;
      }
    }
    lds_barrier();
    // second products: dC, dB per 32 columns; the dx bracket per 32 rows
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      // jobs: 0..NT-1 dC, NT..2NT-1 dB, 2NT, 2NT+1 bracket
      const int j = sl == 0 ? (wave < NT ? wave : (wave < NT + 2 ? 2 * NT + (wave - NT) : -1))
                            : (wave < NT ? NT + wave : -1);
      if (j < 0) continue;
      f32x16 cc;
      if (j < NT) {  // dC(k, n) = e^(l_k) S0^T dy + sum_j W1[k][j] B[j][n]
#pragma unroll
        for (int r = 0; r < 16; ++r) cc[r] = __expf(sm.l[tile_row(r, ln)]) * sm.S0[tile_row(r, ln) * PB + 32 * j + tile_col(ln)];
        mma_tile<kChunk, kPW, 1, PB, 1>(cc, sm.W1, sm.B + 32 * j, ln);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int k = tile_row(r, ln);
          if (k < clen)  // the block's heads added in order
            a.dC_part[((size_t)(c0 + k) * HP + hp) * N + 32 * j + tile_col(ln)] = hh == 0 ? cc[r] : prevC[r] + cc[r];
        }
      } else if (j < 2 * NT) {  // dB(k, n) = dt_k [e^(l_e-l_k) G^T x + sum_m W2[k][m] C[m][n]]
        const int nt = j - NT;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          cc[r] = __expf(le - sm.l[tile_row(r, ln)]) * sm.G[tile_row(r, ln) * PB + 32 * nt + tile_col(ln)];
        mma_tile<kChunk, kPW, 1, PB, 1>(cc, sm.W2, sm.C + 32 * nt, ln);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int k = tile_row(r, ln);
          if (k < clen)
            a.dB_part[((size_t)(c0 + k) * HP + hp) * N + 32 * nt + tile_col(ln)] =
                hh == 0 ? sm.dt[k] * cc[r] : fmaf(sm.dt[k], cc[r], prevB[r]);
        }
      } else {  // bracket(j, p) = e^(l_e-l_j) (G B_j)[p] + sum_k W3[j][k] dy[k][p]; dx = D dy + dt_j bracket
        const int pt = j - 2 * NT;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          cc[r] = __expf(le - sm.l[tile_row(r, ln)]) * sm.GB[tile_row(r, ln) * kPX + 32 * pt + tile_col(ln)];
        mma_tile<kChunk, kPW, 1, kPX, 1>(cc, sm.W3, sm.dy + 32 * pt, ln);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jj = tile_row(r, ln), p = 32 * pt + tile_col(ln);
          sm.GB[jj * kPX + p] = cc[r];  // this wave's own entries: read above, overwritten here
          if (jj < clen)
            a.dx[((size_t)(c0 + jj) * a.H + h) * kHeadDim + p] = fmaf(Dh, sm.dy[jj * kPX + p], sm.dt[jj] * cc[r]);
        }
      }
    }
    lds_barrier();
    // s_j = x_j . bracket_j; then a_i <dS_i, S_{i-1}> -> ddt_i, dA
    {
      const int k = tid >> 4, sub = tid & 15;
      float sv = 0.f;
      for (int p = sub; p < kHeadDim; p += 16) sv = fmaf(sm.x[k * kPX + p], sm.GB[k * kPX + p], sv);
      sv = sum16_dpp(sv);
      // W_k - e^(l_e) <G, S0> = sum_{kk >= k} (Z(kk, k) + q_kk) + sum_{j < k} r'_j
      float wv = 0.f;
      for (int kk = k + sub; kk < kChunk; kk += 16) wv += sm.Z[kk * kPZ + k] + sm.q[kk];
      for (int j = sub; j < k; j += 16) wv += sm.r[j];
      wv = sum16_dpp(wv);
      if (sub == 0) {
        const float W = wv + ele * gs;
        if (k < clen) a.ddt[(size_t)(c0 + k) * a.H + h] = fmaf(Ah, W, sv);
        dA_acc = fmaf(sm.dt[k], W, dA_acc);
      }
    }
    // dy rows scaled by e^(l_k) for the update of G
    for (int e = tid; e < kChunk * kHeadDim; e += kBwdThreads) {
      const int k = e / kHeadDim, p = e % kHeadDim;
      sm.dy[k * kPX + p] *= __expf(sm.l[k]);
    }
    lds_barrier();
    // gradient leaving the previous chunk: G <- e^(l_e) G + sum_k e^(l_k) dy_k outer C_k
    if (gown) {
#pragma unroll
      for (int r = 0; r < 16; ++r) Gt[r] *= ele;
      mma_tile<kChunk, 1, kPX, PB, 1>(Gt, sm.dy + 32 * gp, sm.C + 32 * gn, ln);
    }
    lds_barrier();
  }
  dA_acc = block_sum(dA_acc, sm.red);
  dD_acc = block_sum(dD_acc, sm.red);
  if (tid == 0) {
    a.dA_part[(size_t)u * a.H + h] = dA_acc;
    a.dD_part[(size_t)u * a.H + h] = dD_acc;
  }
}

// one block per (unit, block of hpb heads of one group), the heads in order:
// each adds its dB, dC terms onto the previous head's (every lane writes the
// same entries for every head), so the group sum reads H / hpb partials
template <int N>
__global__ __launch_bounds__(kBwdThreads) void ssm_bwd_grad_kernel(ScanBwdArgs a) {
  __shared__ __attribute__((aligned(16))) BwdSmem<N> sm;
  const int HP = a.H / a.hpb;
  const int u = blockIdx.x / HP, hp = blockIdx.x % HP;
  for (int hh = 0; hh < a.hpb; ++hh) {
    ssm_bwd_grad_head<N>(a, sm, u, hp * a.hpb + hh, hp, hh);
    __syncthreads();  // the next head reuses LDS
  }
}

// dB, dC: the partials of each group summed in head order; one thread per (token, group, column)
__global__ void ssm_bwd_group_sum_kernel(ScanBwdArgs a, int N) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)a.T * a.G * N) return;
  const int n = int(idx % N);
  const long long tg = idx / N;
  const int g = int(tg % a.G);
  const long long t = tg / a.G;
  const int HP = a.H / a.hpb, ppg = a.H / a.G / a.hpb;  // partials per group
  float sb = 0.f, sc = 0.f;
  for (int q = 0; q < ppg; ++q) {
    const size_t off = ((size_t)t * HP + g * ppg + q) * N + n;
    sb += a.dB_part[off];
    sc += a.dC_part[off];
  }
  a.dB[idx] = sb;
  a.dC[idx] = sc;
}

// dA, dD: the units summed in unit order; one thread per head
__global__ void ssm_bwd_unit_sum_kernel(ScanBwdArgs a) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= a.H) return;
  float sa = 0.f, sd = 0.f;
  for (int u = 0; u < a.U; ++u) {
    sa += a.dA_part[(size_t)u * a.H + h];
    sd += a.dD_part[(size_t)u * a.H + h];
  }
  a.dA[h] = sa;
  a.dD[h] = sd;
}

template <int N>
hipError_t launch_ssm_bwd(const ScanBwdArgs& a, hipStream_t s) {
  const dim3 grid(unsigned(a.U) * unsigned(a.H));
  const LocalArgs la{a.dy, a.C, a.dt, a.A, a.unit_start, a.unit_len, a.H, a.G, a.in, a.decay};
  hipLaunchKernelGGL((ssm_unit_local_kernel<N, true>), grid, dim3(kFwdThreads), 0, s, la);
  hipLaunchKernelGGL((ssm_bwd_propagate_kernel<N>), dim3(unsigned(a.H) * 4), dim3(256), 0, s, a);
  hipLaunchKernelGGL((ssm_bwd_grad_kernel<N>), dim3(unsigned(a.U) * unsigned(a.H / a.hpb)), dim3(kBwdThreads), 0,
                     s, a);
  const long long n = (long long)a.T * a.G * N;
  hipLaunchKernelGGL(ssm_bwd_group_sum_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, a, N);
  hipLaunchKernelGGL(ssm_bwd_unit_sum_kernel, dim3(unsigned((a.H + 63) / 64)), dim3(64), 0, s, a);
  return hipGetLastError();
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// heads per block of the gradient pass: 4, 2 or 1, whichever divides the heads of a group
int grad_heads_per_block(const tree_attn_ssm_shape* shape) {
  const int hpg = shape->num_heads / shape->num_groups;
  return hpg % 4 == 0 ? 4 : hpg % 2 == 0 ? 2 : 1;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_plan(const char* fn, tree_attn_mamba_plan_t plan) {
  if (!plan) return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": plan is NULL");
  if (plan->device < 0)
    return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": plan was built host-only");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->device)
    return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": plan was built on another device");
  return TREE_ATTN_OK;
}

// the caller's token count must be the plan's: every kernel walks plan->T rows
int check_tokens(const char* fn, const tree_attn_mamba_plan_s* p, int32_t num_tokens) {
  if (num_tokens != p->T)
    return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": num_tokens " + std::to_string(num_tokens) +
                                                        " != plan tokens " + std::to_string(p->T));
  return TREE_ATTN_OK;
}

int check_ssm_shape(const char* fn, const tree_attn_mamba_plan_s* p, const tree_attn_ssm_shape* sh) {
  const std::string f(fn);
  if (!sh) return report_error(TREE_ATTN_INVALID_ARGUMENT, f + ": shape is NULL");
  if (int rc = check_tokens(fn, p, sh->num_tokens)) return rc;
  if (sh->num_heads < 1 || sh->num_groups < 1 || sh->num_heads % sh->num_groups != 0)
    return report_error(TREE_ATTN_UNSUPPORTED, f + ": num_heads must be a positive multiple of num_groups");
  if (sh->head_dim != kHeadDim)
    return report_error(TREE_ATTN_UNSUPPORTED, f + ": head_dim must be 64");
  if (sh->state_dim != 64 && sh->state_dim != 128)
    return report_error(TREE_ATTN_UNSUPPORTED, f + ": state_dim must be 64 or 128");
  return TREE_ATTN_OK;
}

size_t state_floats(const tree_attn_mamba_plan_s* p, const tree_attn_ssm_shape* sh) {
  return size_t(p->U) * sh->num_heads * sh->head_dim * sh->state_dim;
}

size_t saved_state_floats(const tree_attn_mamba_plan_s* p, const tree_attn_ssm_shape* sh) {
  return state_floats(p, sh) * kChunksPerUnit;
}

int hip_error(const char* fn, hipError_t e) {
  return report_error(TREE_ATTN_HIP_ERROR, std::string(fn) + ": " + hipGetErrorString(e));
}

}  // namespace

extern "C" {

static int mamba_plan_impl(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                           int32_t num_segments, bool upload, tree_attn_mamba_plan_t* out, const char* fn) {
  if (!out) return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": out is NULL");
  *out = nullptr;
  if (!parent || !seg_start || !seg_len)
    return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": NULL topology array");
  return tree_attn::guard_host(fn, [&]() -> int {
    auto m = std::make_unique<tree_attn_mamba_plan_s>();
    std::string err;
    if (!tree_attn::build_mamba_tables(parent, seg_start, seg_len, num_segments, *m, err))
      return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": " + err);
    if (upload) {
      if (hipError_t e = upload_mamba_plan(*m); e != hipSuccess) {
        if (m->block) (void)hipFree(m->block);
        return hip_error(fn, e);
      }
    }
    *out = m.release();
    return TREE_ATTN_OK;
  });
}

int tree_attn_mamba_plan(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                         int32_t num_segments, tree_attn_mamba_plan_t* out) {
  return mamba_plan_impl(parent, seg_start, seg_len, num_segments, true, out, "tree_attn_mamba_plan");
}

int tree_attn_mamba_plan_host(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                              int32_t num_segments, tree_attn_mamba_plan_t* out) {
  return mamba_plan_impl(parent, seg_start, seg_len, num_segments, false, out, "tree_attn_mamba_plan_host");
}

int tree_attn_mamba_plan_destroy(tree_attn_mamba_plan_t plan) {
  if (!plan) return TREE_ATTN_OK;
  if (plan->block) {
    int prev = -1;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(plan->device);
    (void)hipFree(plan->block);
    if (prev >= 0) (void)hipSetDevice(prev);
  }
  delete plan;
  return TREE_ATTN_OK;
}

int tree_attn_mamba_plan_info(tree_attn_mamba_plan_t plan, tree_attn_mamba_plan_info_t* info) {
  if (!plan || !info) return report_error(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_mamba_plan_info: NULL argument");
  info->num_tokens = plan->T;
  info->num_segments = plan->S;
  info->num_units = plan->U;
  info->unit_tokens = kUnit;
  info->max_depth = plan->max_depth;
  info->max_conv_width = kConvMaxWidth;
  return TREE_ATTN_OK;
}

int tree_attn_mamba_plan_export(tree_attn_mamba_plan_t plan, int32_t which, int32_t* buf, int64_t cap,
                                int64_t* count) {
  if (!plan || !count)
    return report_error(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_mamba_plan_export: NULL argument");
  const std::vector<int32_t>* v = nullptr;
  switch (which) {
    case TREE_ATTN_MAMBA_PREV: v = &plan->prev; break;
    case TREE_ATTN_MAMBA_UNIT_START: v = &plan->unit_start; break;
    case TREE_ATTN_MAMBA_UNIT_LEN: v = &plan->unit_len; break;
    case TREE_ATTN_MAMBA_UNIT_PRED: v = &plan->unit_pred; break;
    default: return report_error(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_mamba_plan_export: unknown table");
  }
  *count = int64_t(v->size());
  if (buf) {
    if (cap < *count) return report_error(TREE_ATTN_INVALID_ARGUMENT, "tree_attn_mamba_plan_export: buffer too small");
    std::memcpy(buf, v->data(), v->size() * 4);
  }
  return TREE_ATTN_OK;
}

int tree_attn_conv_fwd(const float* x, const float* weight, const float* bias, int32_t num_tokens,
                       int32_t channels, int32_t width, tree_attn_mamba_plan_t plan, float* y, void* stream) {
  const char* fn = "tree_attn_conv_fwd";
  if (int rc = check_plan(fn, plan)) return rc;
  if (int rc = check_tokens(fn, plan, num_tokens)) return rc;
  if (!x || !weight || !bias || !y) return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": NULL pointer");
  if (channels < 4 || channels % 4 != 0)
    return report_error(TREE_ATTN_UNSUPPORTED, std::string(fn) + ": channels must be a positive multiple of 4");
  if (width < 1 || width > kConvMaxWidth)
    return report_error(TREE_ATTN_UNSUPPORTED, std::string(fn) + ": width must be 1..4");
  if (!aligned16(x) || !aligned16(bias) || !aligned16(y) || !aligned16(weight))
    return report_error(TREE_ATTN_INVALID_ARGUMENT,
                        std::string(fn) + ": x, weight, bias and y must be 16-byte aligned");
  const int C4 = channels / 4;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>((plan->T + kConvTokens - 1) / kConvTokens),
                  static_cast<unsigned>((C4 + 255) / 256)),
      block(256);
  const float4* x4 = reinterpret_cast<const float4*>(x);
  const float4* b4 = reinterpret_cast<const float4*>(bias);
  float4* y4 = reinterpret_cast<float4*>(y);
  switch (width) {
    case 1: hipLaunchKernelGGL(conv_fwd_kernel<1>, grid, block, 0, s, x4, weight, b4, plan->d_halo, plan->T, C4, y4); break;
    case 2: hipLaunchKernelGGL(conv_fwd_kernel<2>, grid, block, 0, s, x4, weight, b4, plan->d_halo, plan->T, C4, y4); break;
    case 3: hipLaunchKernelGGL(conv_fwd_kernel<3>, grid, block, 0, s, x4, weight, b4, plan->d_halo, plan->T, C4, y4); break;
    default: hipLaunchKernelGGL(conv_fwd_kernel<4>, grid, block, 0, s, x4, weight, b4, plan->d_halo, plan->T, C4, y4); break;
  }
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return hip_error(fn, e);
  return TREE_ATTN_OK;
}

size_t tree_attn_conv_bwd_workspace_bytes(tree_attn_mamba_plan_t plan, int32_t channels, int32_t width) {
  (void)width;
  if (!plan || channels < 1) return 0;
  const size_t nblk = (size_t(plan->T) + kConvRows - 1) / kConvRows;
  return align256(nblk * size_t(channels) * (kConvMaxWidth + 1) * 4);
}

int tree_attn_conv_bwd(const float* x, const float* weight, const float* dy, int32_t num_tokens, int32_t channels,
                       int32_t width, tree_attn_mamba_plan_t plan, float* dx, float* dweight, float* dbias,
                       void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "tree_attn_conv_bwd";
  if (int rc = check_plan(fn, plan)) return rc;
  if (int rc = check_tokens(fn, plan, num_tokens)) return rc;
  if (!x || !weight || !dy || !dx || !dweight || !dbias || !workspace)
    return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": NULL pointer");
  if (channels < 4 || channels % 4 != 0)
    return report_error(TREE_ATTN_UNSUPPORTED, std::string(fn) + ": channels must be a positive multiple of 4");
  if (width < 1 || width > kConvMaxWidth)
    return report_error(TREE_ATTN_UNSUPPORTED, std::string(fn) + ": width must be 1..4");
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dx) || !aligned16(weight))
    return report_error(TREE_ATTN_INVALID_ARGUMENT,
                        std::string(fn) + ": x, dy, dx and weight must be 16-byte aligned");
  const size_t need = tree_attn_conv_bwd_workspace_bytes(plan, channels, width);
  if (workspace_bytes < need)
    return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": workspace " +
                                                        std::to_string(workspace_bytes) + " bytes < required " +
                                                        std::to_string(need));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int C4 = channels / 4, T = plan->T;
  {
    const dim3 grid(static_cast<unsigned>((T + kConvTokens - 1) / kConvTokens), static_cast<unsigned>((C4 + 255) / 256)),
        block(256);
    const float4* g4 = reinterpret_cast<const float4*>(dy);
    float4* d4 = reinterpret_cast<float4*>(dx);
    const int32_t *cp = plan->d_csucc_ptr, *cs = plan->d_csucc;
    switch (width) {
      case 1: hipLaunchKernelGGL(conv_bwd_dx_kernel<1>, grid, block, 0, s, g4, weight, plan->d_halo, cp, cs, T, C4, d4); break;
      case 2: hipLaunchKernelGGL(conv_bwd_dx_kernel<2>, grid, block, 0, s, g4, weight, plan->d_halo, cp, cs, T, C4, d4); break;
      case 3: hipLaunchKernelGGL(conv_bwd_dx_kernel<3>, grid, block, 0, s, g4, weight, plan->d_halo, cp, cs, T, C4, d4); break;
      default: hipLaunchKernelGGL(conv_bwd_dx_kernel<4>, grid, block, 0, s, g4, weight, plan->d_halo, cp, cs, T, C4, d4); break;
    }
  }
  const int nblk = (T + kConvRows - 1) / kConvRows;
  float* partial = static_cast<float*>(workspace);
  hipLaunchKernelGGL(conv_bwd_dw_partial_kernel, dim3(unsigned(nblk), unsigned((C4 + 63) / 64)), dim3(64), 0, s,
                     reinterpret_cast<const float4*>(x), reinterpret_cast<const float4*>(dy), plan->d_halo, T, C4,
                     width, partial);
  hipLaunchKernelGGL(conv_bwd_dw_reduce_kernel, dim3(unsigned((channels + 255) / 256)), dim3(256), 0, s, partial,
                     nblk, channels, width, dweight, dbias);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return hip_error(fn, e);
  return TREE_ATTN_OK;
}

size_t tree_attn_ssm_states_bytes(tree_attn_mamba_plan_t plan, const tree_attn_ssm_shape* shape) {
  if (!plan || !shape || shape->num_heads < 1 || shape->head_dim < 1 || shape->state_dim < 1) return 0;
  return align256(saved_state_floats(plan, shape) * 4);
}

size_t tree_attn_ssm_workspace_bytes(tree_attn_mamba_plan_t plan, const tree_attn_ssm_shape* shape) {
  if (!plan || !shape || shape->num_heads < 1 || shape->head_dim < 1 || shape->state_dim < 1) return 0;
  return align256(state_floats(plan, shape) * 4) + align256(size_t(plan->U) * shape->num_heads * 4);
}

size_t tree_attn_ssm_bwd_workspace_bytes(tree_attn_mamba_plan_t plan, const tree_attn_ssm_shape* shape) {
  if (!plan || !shape || shape->num_heads < 1 || shape->num_groups < 1 || shape->head_dim < 1 ||
      shape->state_dim < 1)
    return 0;
  const size_t st = align256(state_floats(plan, shape) * 4);
  const size_t part = align256(size_t(plan->T) * (shape->num_heads / grad_heads_per_block(shape)) *
                               shape->state_dim * 4);
  const size_t uh = align256(size_t(plan->U) * shape->num_heads * 4);
  return 2 * st + 2 * part + 3 * uh;
}

int tree_attn_ssm_bwd(const float* x, const float* dt, const float* A, const float* B, const float* C,
                      const float* D, const float* dy, tree_attn_mamba_plan_t plan, const tree_attn_ssm_shape* shape,
                      const float* states, size_t states_bytes, float* dx, float* ddt, float* dA, float* dB,
                      float* dC, float* dD, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "tree_attn_ssm_bwd";
  if (int rc = check_plan(fn, plan)) return rc;
  if (int rc = check_ssm_shape(fn, plan, shape)) return rc;
  if (!x || !dt || !A || !B || !C || !D || !dy || !states || !dx || !ddt || !dA || !dB || !dC || !dD || !workspace)
    return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": NULL pointer");
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dx) || !aligned16(B) || !aligned16(C) || !aligned16(states) ||
      !aligned16(workspace))
    return report_error(TREE_ATTN_INVALID_ARGUMENT,
                        std::string(fn) + ": x, dy, dx, B, C, states and workspace must be 16-byte aligned");
  if (states_bytes < tree_attn_ssm_states_bytes(plan, shape))
    return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": states buffer too small");
  if (workspace_bytes < tree_attn_ssm_bwd_workspace_bytes(plan, shape))
    return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": workspace too small");
  if ((long long)plan->U * shape->num_heads >= (1LL << 31) ||
      (long long)plan->T * shape->num_groups * shape->state_dim >= (1LL << 40))
    return report_error(TREE_ATTN_UNSUPPORTED, std::string(fn) + ": too many units x heads");
  ScanBwdArgs a{};
  a.x = x, a.dt = dt, a.A = A, a.B = B, a.C = C, a.D = D, a.dy = dy, a.states = states;
  a.unit_start = plan->d_unit_start, a.unit_len = plan->d_unit_len, a.unit_pred = plan->d_unit_pred;
  a.usucc_ptr = plan->d_usucc_ptr, a.usucc = plan->d_usucc, a.uchain = plan->d_uchain;
  a.H = shape->num_heads, a.G = shape->num_groups, a.U = plan->U, a.T = plan->T;
  char* w = static_cast<char*>(workspace);
  a.hpb = grad_heads_per_block(shape);
  const size_t st = align256(state_floats(plan, shape) * 4);
  const size_t part = align256(size_t(plan->T) * (shape->num_heads / a.hpb) * shape->state_dim * 4);
  const size_t uh = align256(size_t(plan->U) * shape->num_heads * 4);
  a.in = reinterpret_cast<float*>(w);
  a.gout = reinterpret_cast<float*>(w + st);
  a.dB_part = reinterpret_cast<float*>(w + 2 * st);
  a.dC_part = reinterpret_cast<float*>(w + 2 * st + part);
  a.decay = reinterpret_cast<float*>(w + 2 * st + 2 * part);
  a.dA_part = reinterpret_cast<float*>(w + 2 * st + 2 * part + uh);
  a.dD_part = reinterpret_cast<float*>(w + 2 * st + 2 * part + 2 * uh);
  a.dx = dx, a.ddt = ddt, a.dA = dA, a.dB = dB, a.dC = dC, a.dD = dD;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = shape->state_dim == 128 ? launch_ssm_bwd<128>(a, s) : launch_ssm_bwd<64>(a, s);
  if (e != hipSuccess) return hip_error(fn, e);
  return TREE_ATTN_OK;
}

int tree_attn_ssm_fwd(const float* x, const float* dt, const float* A, const float* B, const float* C,
                      const float* D, tree_attn_mamba_plan_t plan, const tree_attn_ssm_shape* shape, float* y,
                      float* states, size_t states_bytes, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "tree_attn_ssm_fwd";
  if (int rc = check_plan(fn, plan)) return rc;
  if (int rc = check_ssm_shape(fn, plan, shape)) return rc;
  if (!x || !dt || !A || !B || !C || !D || !y || !states || !workspace)
    return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": NULL pointer");
  if (!aligned16(x) || !aligned16(y) || !aligned16(B) || !aligned16(C) || !aligned16(states) ||
      !aligned16(workspace))
    return report_error(TREE_ATTN_INVALID_ARGUMENT,
                        std::string(fn) + ": x, y, B, C, states and workspace must be 16-byte aligned");
  if (states_bytes < tree_attn_ssm_states_bytes(plan, shape))
    return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": states buffer too small");
  if (workspace_bytes < tree_attn_ssm_workspace_bytes(plan, shape))
    return report_error(TREE_ATTN_INVALID_ARGUMENT, std::string(fn) + ": workspace too small");
  if ((long long)plan->U * shape->num_heads >= (1LL << 31))
    return report_error(TREE_ATTN_UNSUPPORTED, std::string(fn) + ": too many units x heads");
  ScanArgs a{};
  a.x = x, a.dt = dt, a.A = A, a.B = B, a.C = C, a.D = D;
  a.unit_start = plan->d_unit_start, a.unit_len = plan->d_unit_len, a.unit_pred = plan->d_unit_pred;
  a.H = shape->num_heads, a.G = shape->num_groups, a.U = plan->U;
  a.y = y;
  a.states = states;
  a.local = static_cast<float*>(workspace);
  a.decay = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(state_floats(plan, shape) * 4));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = shape->state_dim == 128 ? launch_ssm_fwd<128>(a, s) : launch_ssm_fwd<64>(a, s);
  if (e != hipSuccess) return hip_error(fn, e);
  return TREE_ATTN_OK;
}

}  // extern "C"
