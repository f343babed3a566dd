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
//   1. rowstat: delta[h,i] = sum_d dout[i,h,d] * out[i,h,d];
//   2. dkdv (key-major): a workgroup owns 64 keys of one segment and one
//      key/value head; in DFS pre-order the queries that see key j are the
//      contiguous range [j, subtree_end(seg(j))), so it loops over that range
//      (all G query heads) and accumulates dK, dV in registers:
//        S = Q K^T, P = exp(S - lse), dV^T += dO^T P,
//        dP = dO V^T, dS = P (dP - delta), dK^T += Q^T dS;
//   3. dq (query-major): the forward's walk over the ancestor path,
//        S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - delta),
//        dQ^T += K^T dS^T.
#include "kernel_common.hpp"

namespace tree_attn {

// ---------------------------------------------------------------------------
// 1. row statistics

template <typename T, int D>
__global__ __launch_bounds__(256) void tree_attn_rowstat_kernel(const T* __restrict__ out,
                                                                const T* __restrict__ dout,
                                                                float* __restrict__ delta, int T_, int Hq) {
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
    delta[(size_t)h * T_ + i] = acc;
  }
}

// ---------------------------------------------------------------------------
// 2. dK / dV, key-major

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void tree_attn_dkdv_kernel(BwdArgs a) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  using quad = typename M::quad;
  constexpr int BM = 64;               // queries per step
  constexpr int E = Chunk<T>::E;
  constexpr int CPR = D / E;
  constexpr int KPT = BM * CPR / 256;  // query rows each thread loads per step
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int KSTR = D + E;
  constexpr int QSTR = BM + 4;
  static_assert(KPT == 4, "tile loader assumes 4 rows per thread");
  constexpr int kTileElems = BM * KSTR;  // sQ, sdO
  constexpr int kTElems = D * QSTR;      // sQt, sdOt
  constexpr int kLdsBytes = (2 * kTileElems + 2 * kTElems) * int(sizeof(T));
  constexpr int kRedBytes = 2 * (2 * DB * 16) * 64 * 4;  // two waves' dK/dV partials
  static_assert(kRedBytes <= kLdsBytes, "reduction buffer aliases the tiles");

  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
  __shared__ float slse[BM], sdelta[BM];
  T* sQ = reinterpret_cast<T*>(lds);
  T* sdO = sQ + kTileElems;
  T* sQt = sdO + kTileElems;
  T* sdOt = sQt + kTElems;

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
  const T* __restrict__ k = static_cast<const T*>(a.k);
  const T* __restrict__ v = static_cast<const T*>(a.v);
  const T* __restrict__ dout = static_cast<const T*>(a.dout);

  frag kf[KS], vf[KS];
  {
    const size_t off = ((size_t)ktok * a.Hkv + g) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = load_frag<T>(k + off + ks * 16);
      vf[ks] = load_frag<T>(v + off + ks * 16);
    }
  }
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  const int dc = tid % CPR, qg = tid / CPR;

  for (int hi = 0; hi < a.G; ++hi) {
    const int h = g * a.G + hi;
    for (int i0 = tile.k0; i0 < tile.qend; i0 += BM) {
      Chunk<T> qc[KPT], oc[KPT];
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        const int qi = i0 + qg * KPT + r;
        if (qi < tile.qend) {
          const size_t off = ((size_t)qi * a.Hq + h) * D + dc * E;
          qc[r] = load_chunk<T>(q + off);
          oc[r] = load_chunk<T>(dout + off);
        } else {
          qc[r] = zero_chunk<T>();
          oc[r] = zero_chunk<T>();
        }
      }
      float lv = 0.f, dl = 0.f;
      if (tid < BM) {
        const int qi = i0 + tid;
        if (qi < tile.qend) {
          lv = a.lse[(size_t)h * a.T + qi] * kLog2e;
          dl = a.delta[(size_t)h * a.T + qi];
        }
      }
      __syncthreads();  // previous step finished with the tiles
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        store_chunk<T>(&sQ[(qg * KPT + r) * KSTR + dc * E], qc[r]);
        store_chunk<T>(&sdO[(qg * KPT + r) * KSTR + dc * E], oc[r]);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        quad tq, to;
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
          tq[r] = qc[r].elem(e);
          to[r] = oc[r].elem(e);
        }
        *reinterpret_cast<quad*>(&sQt[(dc * E + e) * QSTR + qg * KPT]) = tq;
        *reinterpret_cast<quad*>(&sdOt[(dc * E + e) * QSTR + qg * KPT]) = to;
      }
      if (tid < BM) {
        slse[tid] = lv;
        sdelta[tid] = dl;
      }
      __syncthreads();

      // S = Q K^T and dP = dO V^T for this wave's 32 queries x 32 keys
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        M::mma(s, load_frag<T>(&sQ[(qh * 32 + col) * KSTR + ks * 16 + half * 8]), kf[ks]);
        M::mma(dp, load_frag<T>(&sdO[(qh * 32 + col) * KSTR + ks * 16 + half * 8]), vf[ks]);
      }
      const bool need_mask = i0 + qh * 32 < tile.k0 + kb * 32 + 31;
      frag pf[2], dsf[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qr = qh * 32 + c_row(i, half);
        float p = __builtin_amdgcn_exp2f(s[i] * c - slse[qr]);
        if (need_mask && i0 + qr < jkey) p = 0.f;
        const float ds = p * (dp[i] - sdelta[qr]);
        pf[i >> 3][i & 7] = to_elem<T>(p);
        dsf[i >> 3][i & 7] = to_elem<T>(ds);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int o = (db * 32 + col) * QSTR + qh * 32 + 16 * hh + 4 * half;
          M::mma(dv[db], load_frag_split<T>(&sdOt[o]), pf[hh]);
          M::mma(dk[db], load_frag_split<T>(&sQt[o]), dsf[hh]);
        }
    }
  }

  // fixed-order reduction of the two query halves, then one store per key
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);
  constexpr int kVals = 2 * DB * 16;
  if (qh == 1) {
    float* r = red + (size_t)kb * kVals * 64;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        r[(db * 16 + i) * 64 + lane] = dk[db][i];
        r[((DB + db) * 16 + i) * 64 + lane] = dv[db][i];
      }
  }
  __syncthreads();
  if (qh == 0 && key_valid) {
    const float* r = red + (size_t)kb * kVals * 64;
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
          tk[e] = to_elem<T>((dk[db][i] + r[(db * 16 + i) * 64 + lane]) * a.scale);
          tv[e] = to_elem<T>(dv[db][i] + r[((DB + db) * 16 + i) * 64 + lane]);
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
  constexpr int E = Chunk<T>::E;
  constexpr int CPR = D / E;
  constexpr int KPT = BN * CPR / 256;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int KSTR = D + E;
  constexpr int VSTR = BN + 4;
  static_assert(KPT == 4, "tile loader assumes 4 keys per thread");

  __shared__ __attribute__((aligned(16))) T sK[BN * KSTR];
  __shared__ __attribute__((aligned(16))) T sV[BN * KSTR];
  __shared__ __attribute__((aligned(16))) T sKt[D * VSTR];

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

  const T* __restrict__ q = static_cast<const T*>(a.q);
  const T* __restrict__ k = static_cast<const T*>(a.k);
  const T* __restrict__ v = static_cast<const T*>(a.v);
  const T* __restrict__ dout = static_cast<const T*>(a.dout);

  frag qf[KS], of[KS];
  {
    const size_t off = ((size_t)qtok * a.Hq + h) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = load_frag<T>(q + off + ks * 16);
      of[ks] = load_frag<T>(dout + off + ks * 16);
    }
  }
  const float lse2 = a.lse[(size_t)h * a.T + qtok] * kLog2e;
  const float dlt = a.delta[(size_t)h * a.T + qtok];

  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = f32x16{};

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
    __syncthreads();
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      store_chunk<T>(&sK[(kg * KPT + r) * KSTR + dc * E], kc[r]);
      store_chunk<T>(&sV[(kg * KPT + r) * KSTR + dc * E], vc[r]);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      quad t4;
#pragma unroll
      for (int r = 0; r < KPT; ++r) t4[r] = kc[r].elem(e);
      *reinterpret_cast<quad*>(&sKt[(dc * E + e) * VSTR + kg * KPT]) = t4;
    }
    __syncthreads();

    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int o = (kb * 32 + col) * KSTR + ks * 16 + half * 8;
        M::mma(s[kb], load_frag<T>(&sK[o]), qf[ks]);
        M::mma(dp[kb], load_frag<T>(&sV[o]), of[ks]);
      }
    const bool need_mask = v0 + BN - 1 > wave_pos0;
    frag dsf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = __builtin_amdgcn_exp2f(s[kb][i] * c - lse2);
        if (need_mask && v0 + kb * 32 + c_row(i, half) > qpos) p = 0.f;
        dsf[kb][i >> 3][i & 7] = to_elem<T>(p * (dp[kb][i] - dlt));
      }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          M::mma(dq[db], load_frag_split<T>(&sKt[(db * 32 + col) * VSTR + kb * 32 + 16 * hh + 4 * half]),
                 dsf[kb][hh]);
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
                     static_cast<const T*>(a.out), static_cast<const T*>(a.dout), a.delta, a.T, a.Hq);
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
