// Backward kernels: exact dq, dk, dv of L = sum <dout, out> over the tree.
//
// The draft "feat(hybrid): add opt-in shared-prefix attention and Mamba
// execution" (intro) states that the backward pass accumulates branch
// contributions into the shared prefix: dk/dv of a prefix token sum over
// every query, in every branch below it, that sees the token.  Megatron-LM
// issue "Shared-prefix training with context parallelism for exact agent
// trajectories" (section "Describe the solution you'd like") checkpoints
// per-run attention: nothing but lse is kept from the forward pass, and the
// probabilities are recomputed here.
//
// Three launches, no atomics, every output element written once by one
// workgroup in a fixed order (bitwise reproducible):
//   1. rowstat: delta[h,i] = sum_d dout[i,h,d] * out[i,h,d] and
//      lse2[h,i] = lse[h,i] * log2(e), into the workspace;
//   2. dkdv (key-major): a workgroup owns 64 keys of one segment and one
//      key/value head; in DFS pre-order the queries that see key j are the
//      contiguous range [j, subtree_end(seg(j))), so it loops over that range
//      (all G query heads) and accumulates dK, dV in registers:
//        S = Q K^T, P = exp(S - lse), dV^T += dO^T P,
//        dP = dO V^T, dS = P (dP - delta), dK^T += Q^T dS;
//      the 64-query Q / dO tiles and their lse / delta are copied straight
//      into LDS (two buffers, one barrier per step); Q^T and dO^T fragments
//      come from the transposing LDS load of the same row-major tiles;
//   3. dq (query-major): the forward's walk over the ancestor path,
//        S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - delta),
//        dQ^T += K^T dS^T   (K^T from the transposing LDS load).
#include "kernel_common.hpp"

namespace tree_attn {

// 4-byte-per-lane copy global -> LDS: lane l writes (lds_base + 4 l).
__device__ inline void dma4(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_base, 4, 0, 0);
}

// ---------------------------------------------------------------------------
// 1. row statistics

template <typename T, int D>
__global__ __launch_bounds__(256) void tree_attn_rowstat_kernel(const T* __restrict__ out,
                                                                const T* __restrict__ dout,
                                                                const float* __restrict__ lse,
                                                                float* __restrict__ delta,
                                                                float* __restrict__ lse2, int T_, int Hq) {
  constexpr int E = Chunk<T>::E;
  constexpr int CPR = D / E;
  constexpr int RPB = 256 / CPR;
  static_assert(CPR <= 64 && 64 % CPR == 0, "row chunks must tile a wavefront");
  const int row = blockIdx.x * RPB + threadIdx.x / CPR;  // row = i * Hq + h
  const int c = threadIdx.x % CPR;
  const bool valid = row < T_ * Hq;
  float acc = 0.f;
  if (valid) {
    const Chunk<T> o = load_chunk<T>(out + (size_t)row * D + c * E);
    const Chunk<T> d = load_chunk<T>(dout + (size_t)row * D + c * E);
#pragma unroll
    for (int e = 0; e < E; ++e) acc += float(o.elem(e)) * float(d.elem(e));
  }
#pragma unroll
  for (int off = CPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (valid && c == 0) {
    const int i = row / Hq, h = row % Hq;
    const size_t at = (size_t)h * T_ + i;
    delta[at] = acc;
    lse2[at] = lse[at] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// 2. dK / dV, key-major

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void tree_attn_dkdv_kernel(BwdArgs a) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  using quad = typename M::quad;
  constexpr int BM = 64;  // queries per step
  constexpr int E = 16 / int(sizeof(T));
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = BM * kRowBytes / int(sizeof(T));
  static_assert(D * int(sizeof(T)) == kRowBytes, "one 256-byte row per token");
  static_assert(DB * 16 * 64 * 4 <= TILE * int(sizeof(T)), "one wave's partial fits a tile");

  __shared__ __attribute__((aligned(16))) T sQ0[TILE];
  __shared__ __attribute__((aligned(16))) T sO0[TILE];
  __shared__ __attribute__((aligned(16))) T sQ1[TILE];
  __shared__ __attribute__((aligned(16))) T sO1[TILE];
  __shared__ float sL0[BM], sD0[BM], sL1[BM], sD1[BM];

  int tile_rank, g;
  decode_item(blockIdx.x, a.Hkv, tile_rank, g);
  const KTile tile = a.ktiles[tile_rank];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int kb = wave & 1, qh = wave >> 1;
  const int kl = kb * 32 + col;
  const bool key_valid = kl < tile.nk;
  const int ktok = tile.k0 + min(kl, tile.nk - 1);
  const int jkey = tile.k0 + kl;
  const float c = a.scale * kLog2e;

  const T* __restrict__ q = static_cast<const T*>(a.q);
  const T* __restrict__ dout = static_cast<const T*>(a.dout);
  const float* lse2 = a.delta + (size_t)a.Hq * a.T;

  frag kf[KS], vf[KS];
  {
    const size_t off = ((size_t)ktok * a.Hkv + g) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = load_frag<T>(static_cast<const T*>(a.k) + off + ks * 16);
      vf[ks] = load_frag<T>(static_cast<const T*>(a.v) + off + ks * 16);
    }
  }
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  const int nblk = (tile.qend - tile.k0 + BM - 1) / BM;
  const int n_steps = a.G * nblk;
  int lrow[4], lchunk[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    lrow[r] = (4 * wave + r) * 4 + (lane >> 4);
    lchunk[r] = (lane & 15) ^ swz(lrow[r]);
  }
  // rows past the query range read a valid row and are masked to P = 0
  auto issue = [&](int step, T* sQ, T* sO, float* sL, float* sD) {
    const int h = g * a.G + step / nblk;
    const int i0 = tile.k0 + (step % nblk) * BM;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qi = min(i0 + lrow[r], tile.qend - 1);
      const size_t off = ((size_t)qi * a.Hq + h) * D + lchunk[r] * E;
      dma16(q + off, sQ + (4 * wave + r) * 64 * E);
      dma16(dout + off, sO + (4 * wave + r) * 64 * E);
    }
    if (wave < 2) {
      const size_t at = (size_t)h * a.T + min(i0 + lane, tile.qend - 1);
      dma4(wave == 0 ? lse2 + at : a.delta + at, wave == 0 ? sL : sD);
    }
  };

  auto compute = [&](int step, const T* sQ, const T* sO, const float* sL, const float* sD) {
    const int i0 = tile.k0 + (step % nblk) * BM;
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      M::mma(s, tile_row_frag<T>(sQ, qh * 32 + col, ks * 16 + half * 8), kf[ks]);
      M::mma(dp, tile_row_frag<T>(sO, qh * 32 + col, ks * 16 + half * 8), vf[ks]);
    }
    const bool need_mask = i0 + qh * 32 < tile.k0 + kb * 32 + 31 || i0 + qh * 32 + 31 >= tile.qend;
    frag pf[2], dsf[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int qr = qh * 32 + c_row(i, half);
      float p = __builtin_amdgcn_exp2f(fmaf(s[i], c, -sL[qr]));
      if (need_mask && (i0 + qr < jkey || i0 + qr >= tile.qend)) p = 0.f;
      pf[i >> 3][i & 7] = to_elem<T>(p);
      dsf[i >> 3][i & 7] = to_elem<T>(p * (dp[i] - sD[qr]));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        M::mma(dv[db], tile_tr_frag<T>(sO, qh * 32 + 16 * hh, db * 32, lane), pf[hh]);
        M::mma(dk[db], tile_tr_frag<T>(sQ, qh * 32 + 16 * hh, db * 32, lane), dsf[hh]);
      }
  };

  issue(0, sQ0, sO0, sL0, sD0);
  wait_dma();
  __syncthreads();
  for (int step = 0;;) {
    const bool more1 = step + 1 < n_steps;
    if (more1) issue(step + 1, sQ1, sO1, sL1, sD1);
    compute(step, sQ0, sO0, sL0, sD0);
    if (!more1) break;
    wait_dma();
    __syncthreads();
    ++step;
    const bool more0 = step + 1 < n_steps;
    if (more0) issue(step + 1, sQ0, sO0, sL0, sD0);
    compute(step, sQ1, sO1, sL1, sD1);
    if (!more0) break;
    wait_dma();
    __syncthreads();
    ++step;
  }

  // fixed-order reduction of the two query halves, then one store per key:
  // the qh = 1 waves park their dK (in sQ0 / sO0) and dV (in sQ1 / sO1)
  __syncthreads();
  float* rk = reinterpret_cast<float*>(kb == 0 ? sQ0 : sO0);
  float* rv = reinterpret_cast<float*>(kb == 0 ? sQ1 : sO1);
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        rk[(db * 16 + i) * 64 + lane] = dk[db][i];
        rv[(db * 16 + i) * 64 + lane] = dv[db][i];
      }
  }
  __syncthreads();
  if (qh == 0 && key_valid) {
    T* dkp = static_cast<T*>(a.dk) + ((size_t)jkey * a.Hkv + g) * D;
    T* dvp = static_cast<T*>(a.dv) + ((size_t)jkey * a.Hkv + g) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        quad tk, tv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = grp * 4 + e;
          tk[e] = to_elem<T>((dk[db][i] + rk[(db * 16 + i) * 64 + lane]) * a.scale);
          tv[e] = to_elem<T>(dv[db][i] + rv[(db * 16 + i) * 64 + lane]);
        }
        *reinterpret_cast<quad*>(dkp + db * 32 + grp * 8 + half * 4) = tk;
        *reinterpret_cast<quad*>(dvp + db * 32 + grp * 8 + half * 4) = tv;
      }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ, query-major (same walk as the forward kernel)

template <typename T, int D, int HG>
__global__ __launch_bounds__(256, 2) void tree_attn_dq_kernel(BwdArgs a) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  using quad = typename M::quad;
  constexpr int BN = 64;
  constexpr int E = 16 / int(sizeof(T));
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = BN * kRowBytes / int(sizeof(T));
  static_assert(D * int(sizeof(T)) == kRowBytes, "one 256-byte row per token");

  __shared__ __attribute__((aligned(16))) T sK0[TILE];
  __shared__ __attribute__((aligned(16))) T sV0[TILE];
  __shared__ __attribute__((aligned(16))) T sK1[TILE];
  __shared__ __attribute__((aligned(16))) T sV1[TILE];
  __shared__ Span sSpans[kMaxSpans];

  int tile_rank, group;
  decode_item(blockIdx.x, a.Hq / HG, tile_rank, group);
  const QTile tile = a.qtiles[tile_rank];

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

  const T* kg = static_cast<const T*>(a.k) + (size_t)g * D;
  const T* vg = static_cast<const T*>(a.v) + (size_t)g * D;
  const size_t row_stride = (size_t)a.Hkv * D;

  frag qf[KS], of[KS];
  {
    const size_t off = ((size_t)qtok * a.Hq + h) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = load_frag<T>(static_cast<const T*>(a.q) + off + ks * 16);
      of[ks] = load_frag<T>(static_cast<const T*>(a.dout) + off + ks * 16);
    }
  }
  const float lse2 = a.delta[(size_t)a.Hq * a.T + (size_t)h * a.T + qtok];
  const float dlt = a.delta[(size_t)h * a.T + qtok];

  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = f32x16{};

  stage_spans(sSpans, a.span_ptr, a.spans, tile.seg);
  __syncthreads();
  SpanCursor cur{sSpans, 0};
  int lrow[4], lchunk[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    lrow[r] = (4 * wave + r) * 4 + (lane >> 4);
    lchunk[r] = (lane & 15) ^ swz(lrow[r]);
  }
  auto issue = [&](int v0, T* sK, T* sV) {
    size_t off[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int vk = min(v0 + lrow[r], kv_len - 1);
      off[r] = (size_t)cur.phys(vk) * row_stride + lchunk[r] * E;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      dma16(kg + off[r], sK + (4 * wave + r) * 64 * E);
      dma16(vg + off[r], sV + (4 * wave + r) * 64 * E);
    }
  };

  auto compute = [&](int v0, const T* sK, const T* sV) {
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        M::mma(s[kb], tile_row_frag<T>(sK, kb * 32 + col, ks * 16 + half * 8), qf[ks]);
        M::mma(dp[kb], tile_row_frag<T>(sV, kb * 32 + col, ks * 16 + half * 8), of[ks]);
      }
    const bool need_mask = v0 + BN - 1 > wave_pos0;
    frag dsf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c, -lse2));
        if (need_mask && v0 + kb * 32 + c_row(i, half) > qpos) p = 0.f;
        dsf[kb][i >> 3][i & 7] = to_elem<T>(p * (dp[kb][i] - dlt));
      }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          M::mma(dq[db], tile_tr_frag<T>(sK, kb * 32 + 16 * hh, db * 32, lane), dsf[kb][hh]);
  };

  issue(0, sK0, sV0);
  wait_dma();
  __syncthreads();
  for (int v0 = 0;;) {
    const bool more1 = v0 + BN < kv_len;
    if (more1) issue(v0 + BN, sK1, sV1);
    compute(v0, sK0, sV0);
    if (!more1) break;
    wait_dma();
    __syncthreads();
    v0 += BN;
    const bool more0 = v0 + BN < kv_len;
    if (more0) issue(v0 + BN, sK0, sV0);
    compute(v0, sK1, sV1);
    if (!more0) break;
    wait_dma();
    __syncthreads();
    v0 += BN;
  }

  if (qrow < tile.nq) {
    T* dqp = static_cast<T*>(a.dq) + ((size_t)(tile.q0 + qrow) * a.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        quad t4;
#pragma unroll
        for (int e = 0; e < 4; ++e) t4[e] = to_elem<T>(dq[db][grp * 4 + e] * a.scale);
        *reinterpret_cast<quad*>(dqp + db * 32 + grp * 8 + half * 4) = t4;
      }
  }
}

// ---------------------------------------------------------------------------
// launchers (one per stage; tree_attn_bwd runs all three in order)

template <typename T, int D>
hipError_t launch_bwd_rowstat(const BwdArgs& a, hipStream_t stream) {
  constexpr int CPR = D / Chunk<T>::E;
  constexpr int RPB = 256 / CPR;
  const unsigned rows = (unsigned)a.T * (unsigned)a.Hq;
  hipLaunchKernelGGL((tree_attn_rowstat_kernel<T, D>), dim3((rows + RPB - 1) / RPB), dim3(256), 0, stream,
                     static_cast<const T*>(a.out), static_cast<const T*>(a.dout), a.lse, a.delta,
                     a.delta + (size_t)a.Hq * a.T, a.T, a.Hq);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((tree_attn_dkdv_kernel<T, D>), dim3((unsigned)a.n_ktiles * (unsigned)a.Hkv), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

template <typename T, int D, int HG>
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((tree_attn_dq_kernel<T, D, HG>), dim3((unsigned)a.n_qtiles * (unsigned)(a.Hq / HG)),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

template hipError_t launch_bwd_rowstat<__bf16, 128>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_rowstat<float, 64>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dkdv<__bf16, 128>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dkdv<float, 64>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<__bf16, 128, 1>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<__bf16, 128, 2>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<__bf16, 128, 4>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<float, 64, 1>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<float, 64, 2>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<float, 64, 4>(const BwdArgs&, hipStream_t);

}  // namespace tree_attn
