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
//      (all G query heads) twice, accumulating in registers
//        pass 1: S = Q K^T, P = exp(S - lse), dV^T += dO^T P,
//        pass 2: S, P again, dP = dO V^T, dS = P (dP - delta), dK^T += Q^T dS;
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
//
// The workgroup makes two passes over its query range: the first
// accumulates dV^T += dO^T P, the second dK^T += Q^T dS.  Recomputing S in
// the second pass costs 8 of every 40 MFMA steps, but only one fp32
// accumulator block is live at a time, which keeps two wavefronts per SIMD
// resident (one fused pass needs ~290 registers and runs one wave per SIMD).

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void tree_attn_dkdv_kernel(BwdArgs a) {
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
  __shared__ __attribute__((aligned(16))) float sL0[BM];
  __shared__ __attribute__((aligned(16))) float sD0[BM];
  __shared__ __attribute__((aligned(16))) float sL1[BM];
  __shared__ __attribute__((aligned(16))) float sD1[BM];

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
  const size_t kv_off = ((size_t)ktok * a.Hkv + g) * D + half * 8;

  frag kf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kf[ks] = load_frag<T>(static_cast<const T*>(a.k) + kv_off + ks * 16);

  const int nblk = (tile.qend - tile.k0 + BM - 1) / BM;
  const int n_steps = a.G * nblk;
  int lrow[4], lchunk[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    lrow[r] = (4 * wave + r) * 4 + (lane >> 4);
    lchunk[r] = (lane & 15) ^ swz(lrow[r]);
  }
  // rows past the query range read a valid row and are masked to P = 0
  // element offsets fit in 32 bits (tensors are limited to 2^31 elements)
  auto issue = [&](int step, T* sQ, T* sO, float* sL, float* sD) {
    const int h = g * a.G + step / nblk;
    const int i0 = tile.k0 + (step % nblk) * BM;
    const int last = tile.qend - 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int off = (min(i0 + lrow[r], last) * a.Hq + h) * D + lchunk[r] * E;
      dma16(q + off, sQ + (4 * wave + r) * 64 * E);
      dma16(dout + off, sO + (4 * wave + r) * 64 * E);
    }
    if (wave < 2) {
      const int at = h * a.T + min(i0 + lane, last);
      dma4(wave == 0 ? lse2 + at : a.delta + at, wave == 0 ? sL : sD);
    }
  };

  // lse2 / delta of this lane's 16 C-layout query rows: 4 runs of 4
  auto row_stats = [&](const float* sX, float (&x)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 v4 = *reinterpret_cast<const f32x4*>(sX + qh * 32 + 8 * j + 4 * half);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * j + e] = v4[e];
    }
  };

  // P for this wave's 32 queries x 32 keys, rounded to the input type
  auto probs = [&](int step, const T* sQ, const float* sL, frag (&pf)[2]) {
    const int i0 = tile.k0 + (step % nblk) * BM;
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) M::mma(s, tile_row_frag<T>(sQ, qh * 32 + col, ks * 16 + half * 8), kf[ks]);
    sched_pipeline<kLdsAhead, KS, frag_reads<T>(false)>();
    float lq[16];
    row_stats(sL, lq);
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, -lq[i]));
    // diagonal block (queries before the key) or rows past the range: wave-uniform
    if (__builtin_amdgcn_readfirstlane(int(i0 + qh * 32 < tile.k0 + kb * 32 + 31 ||
                                           i0 + qh * 32 + 31 >= tile.qend))) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = i0 + qh * 32 + c_row(i, half);
        if (qi < jkey || qi >= tile.qend) p[i] = 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) pf[i >> 3][i & 7] = to_elem<T>(p[i]);
  };

  f32x16 acc[DB];
  frag vf[KS];

  // dV pass: dV^T += dO^T P
  auto step_v = [&](int step, const T* sQ, const T* sO, const float* sL, const float*) {
    frag pf[2];
    probs(step, sQ, sL, pf);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        M::mma(acc[db], tile_tr_frag<T>(sO, qh * 32 + 16 * hh, db * 32, lane), pf[hh]);
    sched_pipeline<kLdsAhead, 2 * DB, frag_reads<T>(true)>();
  };
  // dK pass: dP = dO V^T, dS = P (dP - delta), dK^T += Q^T dS; dS uses the
  // same rounded P as the dV pass
  auto step_k = [&](int step, const T* sQ, const T* sO, const float* sL, const float* sD) {
    frag pf[2];
    probs(step, sQ, sL, pf);
    f32x16 dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) M::mma(dp, tile_row_frag<T>(sO, qh * 32 + col, ks * 16 + half * 8), vf[ks]);
    sched_pipeline<kLdsAhead, KS, frag_reads<T>(false)>();
    float dl[16];
    row_stats(sD, dl);
    frag dsf[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) dsf[i >> 3][i & 7] = to_elem<T>(float(pf[i >> 3][i & 7]) * (dp[i] - dl[i]));
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        M::mma(acc[db], tile_tr_frag<T>(sQ, qh * 32 + 16 * hh, db * 32, lane), dsf[hh]);
    sched_pipeline<kLdsAhead, 2 * DB, frag_reads<T>(true)>();
  };

  // one pass over all steps: two statically named buffers, one barrier per step
  auto run = [&](auto&& step_fn) {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
    issue(0, sQ0, sO0, sL0, sD0);
    wait_dma();
    __syncthreads();
    for (int step = 0;;) {
      const bool more1 = step + 1 < n_steps;
      if (more1) issue(step + 1, sQ1, sO1, sL1, sD1);
      step_fn(step, sQ0, sO0, sL0, sD0);
      if (!more1) break;
      wait_dma();
      __syncthreads();
      ++step;
      const bool more0 = step + 1 < n_steps;
      if (more0) issue(step + 1, sQ0, sO0, sL0, sD0);
      step_fn(step, sQ1, sO1, sL1, sD1);
      if (!more0) break;
      wait_dma();
      __syncthreads();
      ++step;
    }
    __syncthreads();  // every wave is done with the tiles
  };

  // fixed-order reduction of the two query halves, then one store per key:
  // the qh = 1 waves park their partial in sQ0 (kb = 0) / sO0 (kb = 1)
  auto reduce_store = [&](T* out, float mul) {
    float* r = reinterpret_cast<float*>(kb == 0 ? sQ0 : sO0);
    if (qh == 1) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) r[(db * 16 + i) * 64 + lane] = acc[db][i];
    }
    __syncthreads();
    if (qh == 0 && key_valid) {
      T* op = out + ((size_t)jkey * a.Hkv + g) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          quad t4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = grp * 4 + e;
            t4[e] = to_elem<T>((acc[db][i] + r[(db * 16 + i) * 64 + lane]) * mul);
          }
          *reinterpret_cast<quad*>(op + db * 32 + grp * 8 + half * 4) = t4;
        }
    }
    __syncthreads();  // the parking buffer is reused by the next pass
  };

  run(step_v);
  reduce_store(static_cast<T*>(a.dv), 1.f);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) vf[ks] = load_frag<T>(static_cast<const T*>(a.v) + kv_off + ks * 16);
  run(step_k);
  reduce_store(static_cast<T*>(a.dk), a.scale);
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
  const int row_stride = a.Hkv * D;

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
  // Row addresses of the 64 keys [v0, v0 + 64).  Spans are usually much
  // longer than a step, so when the whole step lies in one span (checked
  // with a workgroup-uniform cursor) the rows are contiguous from one base;
  // otherwise every lane looks up its own rows.  Rows past the path read
  // any valid row and are masked.  Offsets fit in 32 bits.
  int ucur = 0;
  auto issue = [&](int v0, T* sK, T* sV) {
    while (v0 >= sSpans[ucur].virt + sSpans[ucur].len) ++ucur;
    const int sv = sSpans[ucur].virt, sl = sSpans[ucur].len, spp = sSpans[ucur].phys;
    int off[4];
    if (__builtin_amdgcn_readfirstlane(int(v0 + BN <= sv + sl && v0 + BN <= kv_len))) {
#pragma unroll
      for (int r = 0; r < 4; ++r) off[r] = (spp + (v0 - sv) + lrow[r]) * row_stride + lchunk[r] * E;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) off[r] = cur.phys(min(v0 + lrow[r], kv_len - 1)) * row_stride + lchunk[r] * E;
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
    sched_pipeline<kLdsAhead, 4 * KS, frag_reads<T>(false)>();
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
    sched_pipeline<kLdsAhead, 4 * DB, frag_reads<T>(true)>();
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
