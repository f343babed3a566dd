// Forward kernel: flash-style online-softmax attention of each query tile
// over its segment's ancestor path.
//
// Computes, for every query token i of segment u and query head h,
//   out[i,h] = softmax over V(i) of (scale * q[i,h] . k[j,g]) applied to v[j,g]
//   lse[h,i] = ln sum_{j in V(i)} exp(scale * q[i,h] . k[j,g])
// where V(i) is the ancestor path of u plus u's tokens up to i (Megatron-LM
// issue "Shared-prefix training with context parallelism for exact agent
// trajectories", section "Describe the solution you'd like": attention for
// each query run against only its ancestor path).
//
// Work decomposition (one workgroup = 4 wavefronts):
//   * a workgroup owns a query tile of 32*NT tokens (inside one segment) and
//     HG query heads of one key/value head (NT*HG = 4);
//   * wave w holds 32 query rows (token sub-tile w / HG, head w % HG) with Q
//     in registers;
//   * the workgroup walks the segment's ancestor path as one virtual key
//     sequence (the merged spans of the plan), 64 keys per step: K and V are
//     gathered span by span with 16-byte row-contiguous loads, staged in LDS
//     (K row-major, V transposed), and every wave computes
//       S^T = K Q^T -> online softmax per query column -> O^T += V^T P^T
//     on the matrix cores.  A lane owns one query column, so the row max and
//     row sum are in-lane reductions plus one exchange with lane l ^ 32.
//   * the own-segment causal rule is "virtual key position <= query
//     position", applied only on the last steps of the walk.
#include "kernel_common.hpp"

namespace tree_attn {

template <typename T, int D, int HG>
__global__ __launch_bounds__(256, 2) void tree_attn_fwd_kernel(FwdArgs a) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  using quad = typename M::quad;
  constexpr int BN = 64;                 // keys per step
  constexpr int NT = 4 / HG;             // 32-token sub-tiles per workgroup
  constexpr int E = Chunk<T>::E;         // elements per 16-byte chunk
  constexpr int CPR = D / E;             // chunks per key row
  constexpr int KPT = BN * CPR / 256;    // keys each thread loads per step
  constexpr int KS = D / 16;             // 16-deep steps over head_dim
  constexpr int DB = D / 32;             // 32-row blocks of O^T
  constexpr int KSTR = D + E;            // K row stride in LDS (16-byte pad)
  constexpr int VSTR = BN + 4;           // V^T row stride in LDS
  static_assert(KPT == 4, "tile loader assumes 4 keys per thread");
  static_assert(NT * HG == 4, "four wavefronts per workgroup");

  __shared__ __attribute__((aligned(16))) T sK[BN * KSTR];
  __shared__ __attribute__((aligned(16))) T sVt[D * VSTR];

  int tile_rank, group;
  decode_item(blockIdx.x, a.Hq / HG, tile_rank, group);
  const QTile tile = a.tiles[tile_rank];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int ts = wave / HG;
  const int h = group * HG + wave % HG;
  const int g = h / a.G;
  const int qrow = ts * 32 + col;
  const int qtok = tile.q0 + min(qrow, tile.nq - 1);
  const int qpos = tile.pos0 + qrow;
  const int wave_pos0 = tile.pos0 + ts * 32;
  const int kv_len = tile.pos0 + tile.nq;
  const float c = a.scale * kLog2e;

  const T* __restrict__ q = static_cast<const T*>(a.q);
  const T* __restrict__ k = static_cast<const T*>(a.k);
  const T* __restrict__ v = static_cast<const T*>(a.v);

  frag qf[KS];
  {
    const T* p = q + ((size_t)qtok * a.Hq + h) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = load_frag<T>(p + ks * 16);
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  SpanCursor cur{a.spans + a.span_ptr[tile.seg], 0};
  const int dc = tid % CPR, kg = tid / CPR;
  const size_t row_stride = (size_t)a.Hkv * D;
  const T* kbase = k + (size_t)g * D + dc * E;
  const T* vbase = v + (size_t)g * D + dc * E;

  for (int v0 = 0; v0 < kv_len; v0 += BN) {
    Chunk<T> kc[KPT], vc[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int vk = v0 + kg * KPT + r;
      if (vk < kv_len) {
        const size_t off = (size_t)cur.phys(vk) * row_stride;
        kc[r] = load_chunk<T>(kbase + off);
        vc[r] = load_chunk<T>(vbase + off);
      } else {
        kc[r] = zero_chunk<T>();
        vc[r] = zero_chunk<T>();
      }
    }
    __syncthreads();  // previous step finished reading sK / sVt
#pragma unroll
    for (int r = 0; r < KPT; ++r) store_chunk<T>(&sK[(kg * KPT + r) * KSTR + dc * E], kc[r]);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      quad t4;
#pragma unroll
      for (int r = 0; r < KPT; ++r) t4[r] = vc[r].elem(e);
      *reinterpret_cast<quad*>(&sVt[(dc * E + e) * VSTR + kg * KPT]) = t4;
    }
    __syncthreads();

    // S^T = K Q^T for two 32-key blocks
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        M::mma(s[kb], load_frag<T>(&sK[(kb * 32 + col) * KSTR + ks * 16 + half * 8]), qf[ks]);

    // online softmax (base 2, scale folded in)
    const bool need_mask = v0 + BN - 1 > wave_pos0;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[kb][i] * c;
        if (need_mask && v0 + kb * 32 + c_row(i, half) > qpos) x = -INFINITY;
        s[kb][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    float rs = 0.f;
    frag pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[kb][i] - mnew);
        rs += p;
        pf[kb][i >> 3][i & 7] = to_elem<T>(p);
      }
    l = l * alpha + rs;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          M::mma(o[db], load_frag_split<T>(&sVt[(db * 32 + col) * VSTR + kb * 32 + 16 * hh + 4 * half]),
                 pf[kb][hh]);
  }

  l += __shfl_xor(l, 32);
  if (qrow < tile.nq) {
    const float inv = 1.f / l;
    T* op = static_cast<T*>(a.out) + ((size_t)(tile.q0 + qrow) * a.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        quad t4;
#pragma unroll
        for (int e = 0; e < 4; ++e) t4[e] = to_elem<T>(o[db][grp * 4 + e] * inv);
        *reinterpret_cast<quad*>(op + db * 32 + grp * 8 + half * 4) = t4;
      }
    if (half == 0) a.lse[(size_t)h * a.T + tile.q0 + qrow] = m * kLn2 + __logf(l);
  }
}

template <typename T, int D, int HG>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  const int groups = a.Hq / HG;
  const dim3 grid((unsigned)a.n_tiles * (unsigned)groups);
  hipLaunchKernelGGL((tree_attn_fwd_kernel<T, D, HG>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// explicit instantiations used by the C ABI
template hipError_t launch_fwd<__bf16, 128, 1>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<__bf16, 128, 2>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<__bf16, 128, 4>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<float, 64, 1>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<float, 64, 2>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<float, 64, 4>(const FwdArgs&, hipStream_t);

}  // namespace tree_attn
