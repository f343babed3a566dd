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
//   1. rowstat: -delta[h,i] = -sum_d dout[i,h,d] * out[i,h,d] and
//      -lse2[h,i] = -lse[h,i] * log2(e), into the workspace (negated, so
//      that they enter the products below as initial accumulators or as
//      the addend of a fused multiply-add);
//   2. dkdv (key-major): a workgroup owns 64 keys of one segment and one
//      key/value head; in DFS pre-order the queries that see key j are the
//      contiguous range [j, subtree_end(seg(j))), so it walks that range
//      (all G query heads) once, 64 queries per step; half of its
//      wavefronts form S = Q K^T, P = exp(S - lse) and dV^T += dO^T P, the
//      other half, given P through LDS, dP = dO V^T, dS = P (dP - delta) and
//      dK^T += Q^T dS; the Q / dO tiles and their lse / delta are copied
//      straight into a ring of LDS buffers; Q^T and dO^T fragments come from
//      the transposing LDS load of the same row-major tiles;
//   3. dq (query-major): the forward's walk over the ancestor path,
//        S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - delta),
//        dQ^T += K^T dS^T   (K^T from the transposing LDS load).
#include <atomic>
#include <type_traits>

#include "kernel_common.hpp"

namespace tree_attn {

// ---------------------------------------------------------------------------
// 1. row statistics

template <typename T, int D>
__global__ __launch_bounds__(256) void tree_attn_rowstat_kernel(const T* __restrict__ out,
                                                                const T* __restrict__ dout,
                                                                const float* __restrict__ lse,
                                                                float* __restrict__ ndelta,
                                                                float* __restrict__ nlse2,
                                                                ItemCounters* __restrict__ counters, int T_,
                                                                int Hq, int row0, int row_end) {
  // the later stages hand out their work items through these counters
  if (blockIdx.x == 0 && threadIdx.x < 2 * int(sizeof(ItemCounters) / 4))
    __hip_atomic_store(reinterpret_cast<unsigned*>(counters) + threadIdx.x, 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  constexpr int E = Chunk<T>::E;
  constexpr int CPR = D / E;
  constexpr int RPB = 256 / CPR;
  static_assert(CPR <= 64 && 64 % CPR == 0, "row chunks must tile a wavefront");
  const int row = row0 + blockIdx.x * RPB + threadIdx.x / CPR;  // row = i * Hq + h
  const int c = threadIdx.x % CPR;
  const bool valid = row < row_end;
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
    ndelta[at] = -acc;
    nlse2[at] = -(lse[at] * kLog2e);
  }
}

// ---------------------------------------------------------------------------
// 2. dK / dV, key-major
//
// One 512-thread workgroup per compute unit owns 64 keys of one key/value
// head and walks the query range that sees them (all G query heads), 64
// queries per step, reading the range once.  Its eight wavefronts split by
// role, one of each role per SIMD; within a role, wave bits (kb, qh) pick 32
// keys x 32 queries:
//   * waves 0-3 (dV): S = Q K^T, P = exp2(S c - lse2) rounded to the input
//     type, dV^T += dO^T P, and P is left in LDS (see PHandoff);
//   * waves 4-7 (dK), one step behind: dP = dO V^T, dS = P (dP - delta)
//     with the P of the matching dV wave, dK^T += Q^T dS.
// So S is formed once per step and each SIMD issues the minimum 32 matrix
// products per step.  Q / dO tiles and their lse2 / delta go through rings
// of kRing LDS slots, copied kRing - 2 steps ahead of the dV waves (the dK
// waves hold one more) by the dK waves alone; each of them issues the same
// number of copies per step, so the wait for a step's tiles is a fixed
// count.  One barrier per step orders copies, P hand-off and slot reuse.

template <int N>
using Slot = std::integral_constant<int, N>;

// How a dV wave hands its probabilities to the dK wave of the same block.
// bf16 inputs: P (in [0, 1]) travels as fp16, rounded to nearest -- finer
// than the bf16 operand of dV -- and the dK wave multiplies it into dP -
// delta with a mixed fp16 x fp32 fused multiply-add, with no separate
// conversion; fp32 inputs: P itself.
template <typename T>
struct PHandoff;

template <>
struct PHandoff<__bf16> {
  using frag = Mfma<__bf16>::frag;
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  __device__ static inline frag pack(const frag&, const float* p) {
    h8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (_Float16)p[e];
    return __builtin_bit_cast(frag, v);
  }
  __device__ static inline float times(const frag& f, int e, float x) {
    return __builtin_fmaf((float)__builtin_bit_cast(h8, f)[e], x, 0.f);
  }
};

template <>
struct PHandoff<float> {
  using frag = Mfma<float>::frag;
  __device__ static inline frag pack(const frag& rounded, const float*) { return rounded; }
  __device__ static inline float times(const frag& f, int e, float x) { return f[e] * x; }
};

template <typename T>
struct DkdvRing {
  static constexpr int value = sizeof(T) == 2 ? 4 : 3;  // fits P and the rings in LDS
};

// Wave priorities of the two dK/dV roles.  Both wavefronts of a SIMD (one
// per role) are ready to issue most of the time; issue goes to the oldest
// ready wavefront, which is the dV wave, so its dense vector work (the
// exponentials of P) would hold back the dK wave's products.  Measured per
// phase, the best order is: the dV wave's products first, then the dK
// wave, then the dV wave's vector work, so the dK products run under the dV
// wave's exponentials.
constexpr int kPrioDvProducts = 2;
constexpr int kPrioDk = 1;
constexpr int kPrioDvVector = 0;

// The queries a key tile's walk visits: those of the run that see the tile,
// in two ranges, each walked for every head of the group in turn.  First
// the segment's descendants [send, qend): the same range for every tile of
// the segment, so the tiles of one segment walked at the same time on one
// XCD stay on the same rows, which its L2 then serves once.  Then the
// tile's own segment [qbeg, send), whose length differs from tile to tile.
// An empty first range is dropped; qend is clamped to qbeg when no query of
// the run sees the tile, so neither range has a negative length (the copies
// clamp rows to the range's last row as an unsigned offset).
struct QueryRanges {
  int lo0, hi0, lo1, hi1;
};
__device__ inline QueryRanges query_ranges(const KTile& t, int q_begin, int q_end) {
  const int qbeg = max(t.k0, q_begin), qend = max(min(t.qend, q_end), qbeg);
  const int split = min(max(t.send, qbeg), qend);
  if (split >= qend) return QueryRanges{qbeg, qend, qend, qend};
  return QueryRanges{split, qend, qbeg, split};
}
// steps of `bm` queries per head
__device__ inline int range_blocks(const QueryRanges& r, int bm) {
  return (r.hi0 - r.lo0 + bm - 1) / bm + (r.hi1 - r.lo1 + bm - 1) / bm;
}

// A walk's position: the step's first query, the range [lo, hi) it is in,
// and its head within the group (0 .. G - 1).  Kept incrementally (no
// division).
struct WalkCursor {
  int i0, lo, hi, h;
  __device__ explicit WalkCursor(const QueryRanges& r) : i0(r.lo0), lo(r.lo0), hi(r.hi0), h(0) {}
  __device__ inline void advance(const QueryRanges& r, int G, int bm) {
    i0 += bm;
    if (i0 >= hi) {
      i0 = lo;
      if (++h == G) {  // on to the second range
        h = 0;
        i0 = lo = r.lo1;
        hi = r.hi1;
      }
    }
  }
};

template <typename T, int D>
__device__ __forceinline__ void dkdv_item(const BwdArgs& a, const KTile& tile, int g, char* lds) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  using quad = typename M::quad;
  constexpr int kRing = DkdvRing<T>::value;
  constexpr int kAhead = kRing - 2;               // steps copied ahead
  constexpr int BM = 64;                          // queries per step
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int RB = D * int(sizeof(T));          // bytes of one head's row
  constexpr int TILE = BM * RB;                   // bytes of one 64-row tile
  constexpr int STATS = 2 * BM * 4;               // lse2, delta of one step
  constexpr int NC = path_copies(RB);             // copies per 16 rows
  constexpr int RPC = 1024 / RB;                  // rows per copy
  constexpr int kCopiesK = 2 * NC + 1;            // copies per dK wave per step
  constexpr int PBLK = 2 * 64;                    // P fragments per wave block
  static_assert(RB == 128 || RB == 256, "128- or 256-byte rows");
  static_assert(4 * DB * 16 * 64 * 4 <= 2 * kRing * TILE, "the partials fit the rings");

  // Q ring, then dO ring (each at most 64 KB, so a slot offset fits an LDS
  // immediate), then the lse2 / delta ring
  char* const ring = lds;
  frag (*const pshare)[4 * PBLK] = reinterpret_cast<frag (*)[4 * PBLK]>(lds + 2 * kRing * TILE + kRing * STATS);
  float* const junk = reinterpret_cast<float*>(lds + 2 * kRing * TILE + kRing * STATS + 2 * 4 * PBLK * sizeof(frag));


  // (opaque per item, so nothing derived from the thread index is hoisted
  // out of the item loop to stay live across items)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int col = lane & 31, half = lane >> 5;
  const bool dk_role = wave >= 4;
  const int wblk = wave & 3;
  const int kb = wave & 1, qh = (wave >> 1) & 1;
  const int kl = kb * 32 + col;
  const bool key_valid = kl < tile.nk;
  const int ktok = tile.k0 + min(kl, tile.nk - 1);
  const int jkey = tile.k0 + kl;
  const float c = a.scale * kLog2e;
  const float* lse2 = a.delta + (size_t)a.Hq * a.T;

  // the dV waves keep K, the dK waves V (both as B fragments)
  frag kv[KS];
  {
    const T* src = static_cast<const T*>(dk_role ? a.v : a.k) + ((size_t)ktok * a.Hkv + g) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kv[ks] = load_frag<T>(src + ks * 16);
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) settle(kv[ks]);

  const QueryRanges rg = query_ranges(tile, a.q_begin, a.q_end);
  const int n_steps = a.G * range_blocks(rg, BM);
  if (n_steps == 0) {  // no query of the run sees the tile: zero gradients
    if (qh == 0 && key_valid) {
      T* op = static_cast<T*>(dk_role ? a.dk : a.dv) + ((size_t)jkey * a.Hkv + g) * D;
#pragma unroll
      for (int d = 0; d < D; d += 32)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) *reinterpret_cast<quad*>(op + d + grp * 8 + half * 4) = quad{};
    }
    return;
  }

  const unsigned q_ring = lds_addr(ring), o_ring = q_ring + kRing * TILE, s_ring = q_ring + 2 * kRing * TILE;

  // Copy plan: only the dK waves copy (their vector work, dS with one mixed
  // fma per element, is the lighter: the dV waves carry the exponentials).
  // dK wave w copies rows 16 (w - 4) .. +16 of the Q tile and of the dO
  // tile (NC instructions of 1 KB each) and one 64-float stat vector
  // (waves 4 and 5 the real lse2 / delta, waves 6 and 7 a discarded
  // duplicate): kCopiesK copies per step.  Per lane: row crow0 + RPC r +
  // lane / (RB / 16) and its swizzled 16-byte chunk.
  const int crow0 = wblk * 16;
  const float* ssrc = wave == 5 ? a.delta : lse2;
  const unsigned s_lds = wave == 4 || wave == 5 ? s_ring + (wave - 4) * BM * 4 : lds_addr(junk);
  const unsigned s_step = wave == 4 || wave == 5 ? STATS : 0;
  const int crow = crow0 + lane / (RB / 16);
  const unsigned row_bytes = (unsigned)a.Hq * RB;
  unsigned cchunk[NC], coff[NC];  // swizzled chunk; whole-step offset (row crow + RPC r)
#pragma unroll
  for (int r = 0; r < NC; ++r) {
    cchunk[r] = (((lane % (RB / 16)) ^ swz<RB>(crow + RPC * r)) * 16);
    coff[r] = unsigned(crow + RPC * r) * row_bytes + cchunk[r];
  }
  // Step `step` goes to slot step % kRing.  The copy stream advances one
  // step per call: `cp` is the next step to copy; past the end it stays on
  // the last step, re-copying its rows into the (idle) slot, so a dK wave
  // always issues kCopiesK copies.  Rows past the range read the range's
  // last row (masked to P = 0).  Each copy reads from a wave-uniform row
  // base plus a small per-lane offset.
  int cp_step = 0;
  WalkCursor cp(rg);
  auto issue = [&](int slot) {
    const int cp_i0 = cp.i0, cp_h = g * a.G + cp.h;
    const int lim = cp.hi - 1 - cp_i0;
    const size_t row0 = ((size_t)cp_i0 * a.Hq + cp_h) * D;
    if (lim >= BM - 1) {  // the whole step in range: fixed per-lane offsets
#pragma unroll
      for (int r = 0; r < NC; ++r) {
        const unsigned lofs = crow0 * RB + (unsigned)slot * TILE + RPC * r * RB;
        copy16_async(static_cast<const T*>(a.q) + row0, coff[r], q_ring + lofs);
        copy16_async(static_cast<const T*>(a.dout) + row0, coff[r], o_ring + lofs);
      }
      copy4_async(ssrc + (size_t)cp_h * a.T + cp_i0, (unsigned)lane * 4u, s_lds + (unsigned)slot * s_step);
    } else {
#pragma unroll
      for (int r = 0; r < NC; ++r) {
        const unsigned voff = (unsigned)min(crow + RPC * r, lim) * row_bytes + cchunk[r];
        const unsigned lofs = crow0 * RB + (unsigned)slot * TILE + RPC * r * RB;
        copy16_async(static_cast<const T*>(a.q) + row0, voff, q_ring + lofs);
        copy16_async(static_cast<const T*>(a.dout) + row0, voff, o_ring + lofs);
      }
      copy4_async(ssrc + (size_t)cp_h * a.T + cp_i0, (unsigned)min(lane, lim) * 4u,
                  s_lds + (unsigned)slot * s_step);
    }
    if (++cp_step < n_steps) cp.advance(rg, a.G, BM);
  };

  // Per-lane read addresses in slot 0: A rows (Q for the dV role, dO for
  // the dK role), C transposed (dO, resp. Q), and this lane's stat rows.
  TileAddr<T, D> ta, tc;
  // (the wave's 32-query half of the tile is part of the base, so every
  // read below takes a compile-time offset)
  ta.init((dk_role ? o_ring : q_ring) + qh * 32 * RB, lane);
  tc.init((dk_role ? q_ring : o_ring) + qh * 32 * RB, lane);
  unsigned stat_addr = s_ring + (dk_role ? BM * 4 : 0) + (qh * 32 + 4 * half) * 4;
  asm volatile("" : "+v"(stat_addr));

  // lse2 / delta of this lane's 16 C-layout query rows: 4 runs of 4
  auto row_stats = [&](int off, float (&x)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 v4 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
          (size_t)(stat_addr + off + 32 * j));
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * j + e] = v4[e];
    }
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  // Both roles run every iteration step = 0 .. n_steps without branches
  // (the accumulators stay in place):
  //   dV waves: dV^T += dO^T P of step - 1 (P kept in registers), then
  //             S = Q K^T and P = exp2(S c - lse2) of `step` (zero before
  //             the key or past the range, rounded to the input type, also
  //             left in LDS for the dK waves);
  //   dK waves: dP = dO V^T of step - 1, dS = P (dP - delta) with the dV
  //             waves' P, dK^T += Q^T dS.
  // Each wave thus alternates matrix work with its vector work, and within
  // a SIMD one role's products cover the other role's exp / dS.  Iteration
  // 0 reads a zero-filled slot (kRing - 1) and P buffer, so it adds zero;
  // the S, P of iteration n_steps are never used.
  frag pprev[2];
  WalkCursor dvc(rg);  // the dV waves' current step
  auto dv_iter = [&](int step, auto J) {
    constexpr int j = decltype(J)::value, jp = (j + kRing - 1) % kRing;
    __builtin_amdgcn_s_setprio(kPrioDvProducts);
    // (consecutive products to different accumulators; each sums in the
    // same order)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        M::mma(acc[db], tc.tr(db, jp * TILE + 16 * hh * RB), pprev[hh]);
    f32x16 t = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) M::mma(t, ta.row(ks, j * TILE), kv[ks]);
    // (the dV products take two LDS reads each, the S products one)
    if constexpr (frag_reads<T>(false) > 0)
      sched_products_then_valu<kLdsAhead, 2 * DB, frag_reads<T>(true), KS, frag_reads<T>(false), 0>();
    __builtin_amdgcn_s_setprio(kPrioDvVector);
    float x[16];
    row_stats(j * STATS, x);
    const int i0 = dvc.i0, ihi = dvc.hi;
    dvc.advance(rg, a.G, BM);
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(t[i], c, x[i]));
    if (__builtin_amdgcn_readfirstlane(int(i0 + qh * 32 < tile.k0 + kb * 32 + 31 ||
                                           i0 + qh * 32 + 31 >= ihi))) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = i0 + qh * 32 + c_row(i, half);
        if (qi < jkey || qi >= ihi) p[i] = 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) pprev[i >> 3][i & 7] = to_elem<T>(p[i]);
    frag* pshr = &pshare[step & 1][wblk * PBLK];
    pshr[lane] = PHandoff<T>::pack(pprev[0], p);
    pshr[64 + lane] = PHandoff<T>::pack(pprev[1], p + 8);
  };
  float xd[16];  // -delta of the dK waves' next step (read one iteration early)
#pragma unroll
  for (int i = 0; i < 16; ++i) xd[i] = 0.f;
  auto dk_iter = [&](int step, auto J) {
    constexpr int j = decltype(J)::value, jp = (j + kRing - 1) % kRing;
    __builtin_amdgcn_s_setprio(kPrioDk);
    const frag* pshr = &pshare[(step + 1) & 1][wblk * PBLK];
    const frag pf[2] = {pshr[lane], pshr[64 + lane]};
    // (the P reads go ahead of the software-pipelined fragment reads)
    __builtin_amdgcn_sched_barrier(0);
    // dP - delta: the products accumulate onto -delta
    f32x16 t;
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = xd[i];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) M::mma(t, ta.row(ks, jp * TILE), kv[ks]);
    sched_pipeline<kLdsAhead, KS, frag_reads<T>(false)>();
    frag xf[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) xf[i >> 3][i & 7] = to_elem<T>(PHandoff<T>::times(pf[i >> 3], i & 7, t[i]));
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        M::mma(acc[db], tc.tr(db, jp * TILE + 16 * hh * RB), xf[hh]);
    sched_pipeline<kLdsAhead, 2 * DB, frag_reads<T>(true)>();
    __builtin_amdgcn_sched_barrier(0);
    // -delta of `step` (in LDS since this iteration's barrier; its slot is
    // refilled only kRing - kAhead steps later)
    row_stats(j * STATS, xd);
  };

  // iteration `step` in slot J = step % kRing
  auto body = [&](auto R, int step, auto J) {
    // a dK wave's copies of `step` are done once only the kAhead - 1 newer
    // steps' copies may be in flight; after the barrier every dK wave's are,
    // the P of step - 1 is in LDS, and nobody reads the slot refilled next
    // (last read at step - 2)
    if constexpr (decltype(R)::value) {
      wait_copies_barrier<(kAhead - 1) * kCopiesK>();
      issue((decltype(J)::value + kAhead) % kRing);
      dk_iter(step, J);
    } else {
      wait_copies_barrier<0>();
      dv_iter(step, J);
    }
  };
  // unrolled over the ring slots so every LDS offset is a constant; returns
  // true once iteration n_steps is done
  auto round = [&](auto self, auto R, int step, auto J) -> bool {
    constexpr int j = decltype(J)::value;
    body(R, step + j, J);
    if (step + j >= n_steps) return true;
    if constexpr (j + 1 < kRing) {
      return self(self, R, step, Slot<j + 1>{});
    } else {
      return false;
    }
  };
  // each role runs its own copy of the loop (the same barriers in the same
  // order), so neither role's accumulators are merged with the other's
  auto walk = [&](auto R) {
    for (int step = 0;; step += kRing)
      if (round(round, R, step, Slot<0>{})) break;
  };

  // zero the slot and P buffer that iteration 0 reads, then start copying
  {
    float* z0 = reinterpret_cast<float*>(ring + (kRing - 1) * TILE);              // Q tile
    float* z1 = reinterpret_cast<float*>(ring + (2 * kRing - 1) * TILE);          // dO tile
    for (int i = tid; i < TILE / 4; i += 512) z0[i] = z1[i] = 0.f;
    float* z2 = reinterpret_cast<float*>(ring + 2 * kRing * TILE + (kRing - 1) * STATS);
    if (tid < STATS / 4) z2[tid] = 0.f;
    float* z3 = reinterpret_cast<float*>(&pshare[1][0]);
    for (int i = tid; i < int(sizeof(pshare[1]) / 4); i += 512) z3[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) pprev[0][e] = pprev[1][e] = to_elem<T>(0.f);
  }
  __syncthreads();
  if (dk_role) {
#pragma unroll
    for (int st = 0; st < kAhead; ++st) issue(st);
  }
  if (dk_role)
    walk(std::true_type{});
  else
    walk(std::false_type{});
  __builtin_amdgcn_s_setprio(0);
  wait_copies_barrier<0>();  // no copy in flight; the rings are free

  // fixed-order reduction of the two query halves, then one store per key:
  // the qh = 1 wave of each (role, kb) parks its partial in the ring
  float* park = reinterpret_cast<float*>(ring) + ((dk_role ? 2 : 0) + kb) * (DB * 16 * 64);
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) park[(db * 16 + i) * 64 + lane] = acc[db][i];
  }
  __syncthreads();
  if (qh == 0 && key_valid) {
    T* op = static_cast<T*>(dk_role ? a.dk : a.dv) + ((size_t)jkey * a.Hkv + g) * D;
    const float mul = dk_role ? a.scale : 1.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        quad t4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = grp * 4 + e;
          t4[e] = to_elem<T>((acc[db][i] + park[(db * 16 + i) * 64 + lane]) * mul);
        }
        *reinterpret_cast<quad*>(op + db * 32 + grp * 8 + half * 4) = t4;
      }
  }
}

// LDS of the 64-key walk
template <typename T, int D>
constexpr int dkdv_lds_bytes() {
  constexpr int kRing = DkdvRing<T>::value, TILE = 64 * D * int(sizeof(T));
  return 2 * kRing * TILE + kRing * 2 * 64 * 4 + 2 * 4 * 128 * int(sizeof(typename Mfma<T>::frag)) + 64 * 4;
}

// ---------------------------------------------------------------------------
// 2b. dK / dV over 128-key tiles (bf16)
//
// The 64-key walk above pays a fixed cost per step -- the Q / dO copies, the
// barrier -- for 32 matrix products per SIMD.  Here a workgroup owns 128
// keys and every wavefront takes both 32-query halves of a step, so the same
// 64-query tiles feed twice the products: wavefront w owns keys
// 32 (w mod 4) .. +32 of the tile in its role (dV: waves 0-3, dK: waves
// 4-7, the same per-role work as above) and accumulates both halves itself,
// which also removes the cross-wave reduction at the end.  A step is 64
// products per SIMD, twice as long, so the rings copy one step ahead in
// three slots (about the same lead time as two steps of the 64-key walk) and
// the P hand-off, twice as large, still fits LDS next to them.
template <typename T, int D>
__device__ __forceinline__ void dkdv_wide_item(const BwdArgs& a, const KTile& tile, int g, char* lds) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  using quad = typename M::quad;
  constexpr int kRing = 3;
  constexpr int kAhead = 1;                       // steps copied ahead
  constexpr int BM = 64;                          // queries per step
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int RB = D * int(sizeof(T));          // bytes of one head's row
  constexpr int TILE = BM * RB;                   // bytes of one 64-row tile
  constexpr int STATS = 2 * BM * 4;               // -lse2, -delta of one step
  constexpr int NC = path_copies(RB);             // copies per 16 rows
  constexpr int RPC = 1024 / RB;                  // rows per copy
  constexpr int kCopiesK = 2 * NC + 1;            // copies per dK wave per step
  constexpr int PBLK = 2 * 64;                    // P fragments of one 32 x 32 block
  static_assert(sizeof(T) == 2, "16-bit inputs: the fp32 P hand-off would not fit LDS");
  static_assert(RB == 128 || RB == 256, "128- or 256-byte rows");

  // Q ring, then dO ring, then the -lse2 / -delta ring
  char* const ring = lds;
  frag (*const pshare)[8 * PBLK] = reinterpret_cast<frag (*)[8 * PBLK]>(lds + 2 * kRing * TILE + kRing * STATS);
  float* const junk = reinterpret_cast<float*>(lds + 2 * kRing * TILE + kRing * STATS + 2 * 8 * PBLK * sizeof(frag));


  // (opaque per item, so nothing derived from the thread index is hoisted
  // out of the item loop to stay live across items)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int col = lane & 31, half = lane >> 5;
  const bool dk_role = wave >= 4;
  const int kq = wave & 3;
  const int kl = kq * 32 + col;
  const bool key_valid = kl < tile.nk;
  const int ktok = tile.k0 + min(kl, tile.nk - 1);
  const int jkey = tile.k0 + kl;
  const float c = a.scale * kLog2e;
  const float* nlse2 = a.delta + (size_t)a.Hq * a.T;

  // the dV waves keep K, the dK waves V (both as B fragments)
  frag kv[KS];
  {
    const T* src = static_cast<const T*>(dk_role ? a.v : a.k) + ((size_t)ktok * a.Hkv + g) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kv[ks] = load_frag<T>(src + ks * 16);
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) settle(kv[ks]);

  const QueryRanges rg = query_ranges(tile, a.q_begin, a.q_end);
  const int n_steps = a.G * range_blocks(rg, BM);
  if (n_steps == 0) {  // no query of the run sees the tile: zero gradients
    if (key_valid) {
      T* op = static_cast<T*>(dk_role ? a.dk : a.dv) + ((size_t)jkey * a.Hkv + g) * D;
#pragma unroll
      for (int d = 0; d < D; d += 32)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) *reinterpret_cast<quad*>(op + d + grp * 8 + half * 4) = quad{};
    }
    return;
  }

  const unsigned q_ring = lds_addr(ring), o_ring = q_ring + kRing * TILE, s_ring = q_ring + 2 * kRing * TILE;

  // Copies as in the 64-key walk: dK wave w copies rows 16 (w - 4) .. +16 of
  // the Q and dO tiles and one 64-float stat vector (waves 4 and 5 the real
  // -lse2 / -delta, waves 6 and 7 a discarded duplicate).
  const int crow0 = kq * 16;
  const float* ssrc = wave == 5 ? a.delta : nlse2;
  const unsigned s_lds = wave == 4 || wave == 5 ? s_ring + (wave - 4) * BM * 4 : lds_addr(junk);
  const unsigned s_step = wave == 4 || wave == 5 ? STATS : 0;
  const int crow = crow0 + lane / (RB / 16);
  const unsigned row_bytes = (unsigned)a.Hq * RB;
  unsigned cchunk[NC], coff[NC];  // swizzled chunk; whole-step offset (row crow + RPC r)
#pragma unroll
  for (int r = 0; r < NC; ++r) {
    cchunk[r] = (((lane % (RB / 16)) ^ swz<RB>(crow + RPC * r)) * 16);
    coff[r] = unsigned(crow + RPC * r) * row_bytes + cchunk[r];
  }
  int cp_step = 0;
  WalkCursor cp(rg);
  auto issue = [&](int slot) {
    const int cp_i0 = cp.i0, cp_h = g * a.G + cp.h;
    const int lim = cp.hi - 1 - cp_i0;
    const size_t row0 = ((size_t)cp_i0 * a.Hq + cp_h) * D;
    if (lim >= BM - 1) {  // the whole step in range: fixed per-lane offsets
#pragma unroll
      for (int r = 0; r < NC; ++r) {
        const unsigned lofs = crow0 * RB + (unsigned)slot * TILE + RPC * r * RB;
        copy16_async(static_cast<const T*>(a.q) + row0, coff[r], q_ring + lofs);
        copy16_async(static_cast<const T*>(a.dout) + row0, coff[r], o_ring + lofs);
      }
      copy4_async(ssrc + (size_t)cp_h * a.T + cp_i0, (unsigned)lane * 4u, s_lds + (unsigned)slot * s_step);
    } else {
#pragma unroll
      for (int r = 0; r < NC; ++r) {
        const unsigned voff = (unsigned)min(crow + RPC * r, lim) * row_bytes + cchunk[r];
        const unsigned lofs = crow0 * RB + (unsigned)slot * TILE + RPC * r * RB;
        copy16_async(static_cast<const T*>(a.q) + row0, voff, q_ring + lofs);
        copy16_async(static_cast<const T*>(a.dout) + row0, voff, o_ring + lofs);
      }
      copy4_async(ssrc + (size_t)cp_h * a.T + cp_i0, (unsigned)min(lane, lim) * 4u,
                  s_lds + (unsigned)slot * s_step);
    }
    if (++cp_step < n_steps) cp.advance(rg, a.G, BM);
  };

  // per-lane read addresses in slot 0 (the query half is a constant offset)
  TileAddr<T, D> ta, tc;
  ta.init(dk_role ? o_ring : q_ring, lane);
  tc.init(dk_role ? q_ring : o_ring, lane);
  unsigned stat_addr = s_ring + (dk_role ? BM * 4 : 0) + 4 * half * 4;
  asm volatile("" : "+v"(stat_addr));
  auto row_stats = [&](int off, float (&x)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 v4 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
          (size_t)(stat_addr + off + 32 * j));
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * j + e] = v4[e];
    }
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  // The per-role work of the 64-key walk, for both query halves qh:
  //   dV waves: dV^T += dO^T P of step - 1, then S and P of `step`;
  //   dK waves: dP - delta, dS, dK^T += Q^T dS of step - 1.
  frag pprev[2][2];
  WalkCursor dvc(rg);  // the dV waves' current step
  auto dv_iter = [&](int step, auto J) {
    constexpr int j = decltype(J)::value, jp = (j + kRing - 1) % kRing;
    __builtin_amdgcn_s_setprio(kPrioDvProducts);
    // (consecutive products go to different accumulators; each one still
    // sums in the same order)
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          M::mma(acc[db], tc.tr(db, jp * TILE + (qh * 32 + 16 * hh) * RB), pprev[qh][hh]);
    f32x16 t[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) M::mma(t[qh], ta.row(ks, j * TILE + qh * 32 * RB), kv[ks]);
    // (the dV products take two LDS reads each, the S products one)
    sched_products_then_valu<kLdsAhead, 4 * DB, frag_reads<T>(true), 2 * KS, frag_reads<T>(false), 0>();
    __builtin_amdgcn_s_setprio(kPrioDvVector);
    const int i0 = dvc.i0, ihi = dvc.hi;
    dvc.advance(rg, a.G, BM);
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      float x[16];
      row_stats(j * STATS + qh * 32 * 4, x);
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(t[qh][i], c, x[i]));
      if (__builtin_amdgcn_readfirstlane(int(i0 + qh * 32 < tile.k0 + kq * 32 + 31 ||
                                             i0 + qh * 32 + 31 >= ihi))) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = i0 + qh * 32 + c_row(i, half);
          if (qi < jkey || qi >= ihi) p[i] = 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) pprev[qh][i >> 3][i & 7] = to_elem<T>(p[i]);
      frag* pshr = &pshare[step & 1][(kq * 2 + qh) * PBLK];
      pshr[lane] = PHandoff<T>::pack(pprev[qh][0], p);
      pshr[64 + lane] = PHandoff<T>::pack(pprev[qh][1], p + 8);
    }
  };
  float xd[2][16];  // -delta of the dK waves' next step (read one iteration early)
#pragma unroll
  for (int qh = 0; qh < 2; ++qh)
#pragma unroll
    for (int i = 0; i < 16; ++i) xd[qh][i] = 0.f;
  auto dk_iter = [&](int step, auto J) {
    constexpr int j = decltype(J)::value, jp = (j + kRing - 1) % kRing;
    __builtin_amdgcn_s_setprio(kPrioDk);
    frag pf[2][2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      const frag* pshr = &pshare[(step + 1) & 1][(kq * 2 + qh) * PBLK];
      pf[qh][0] = pshr[lane];
      pf[qh][1] = pshr[64 + lane];
    }
    // (the P reads go ahead of the software-pipelined fragment reads)
    __builtin_amdgcn_sched_barrier(0);
    // dP - delta: the products accumulate onto -delta
    f32x16 t[2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
#pragma unroll
      for (int i = 0; i < 16; ++i) t[qh][i] = xd[qh][i];
    // dP of half 0, then dP of half 1 with half 0's dS between its
    // products, then dK of half 0 with half 1's dS between its products,
    // then dK of half 1: each half's vector work issues while the matrix
    // core works through independent products (same sums, same order)
    frag xf[2][2];
    auto ds = [&](int qh) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        xf[qh][i >> 3][i & 7] = to_elem<T>(PHandoff<T>::times(pf[qh][i >> 3], i & 7, t[qh][i]));
    };
    auto dk = [&](int qh) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          M::mma(acc[db], tc.tr(db, jp * TILE + (qh * 32 + 16 * hh) * RB), xf[qh][hh]);
    };
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) M::mma(t[qh], ta.row(ks, jp * TILE + qh * 32 * RB), kv[ks]);
    ds(0);
    // (operand reads two products ahead here: measured faster than three)
    sched_products_then_valu<2, KS, frag_reads<T>(false), KS, frag_reads<T>(false), 3>();
    __builtin_amdgcn_sched_barrier(0);
    dk(0);
    ds(1);
    dk(1);
    sched_products_then_valu<2, 2 * DB, frag_reads<T>(true), 2 * DB, frag_reads<T>(true), 0, 3>();
    __builtin_amdgcn_sched_barrier(0);
    // -delta of `step` (in LDS since this iteration's barrier; its slot is
    // refilled only kRing - kAhead steps later)
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) row_stats(j * STATS + qh * 32 * 4, xd[qh]);
  };

  // iteration `step` in slot J = step % kRing; at its barrier every dK
  // wave's copies of `step` are in LDS, the P of step - 1 is in LDS, and
  // nobody reads the slot refilled next (last read at step - 2)
  auto body = [&](auto R, int step, auto J) {
    if constexpr (decltype(R)::value) {
      wait_copies_barrier<(kAhead - 1) * kCopiesK>();
      issue((decltype(J)::value + kAhead) % kRing);
      dk_iter(step, J);
    } else {
      wait_copies_barrier<0>();
      dv_iter(step, J);
    }
  };
  auto round = [&](auto self, auto R, int step, auto J) -> bool {
    constexpr int j = decltype(J)::value;
    body(R, step + j, J);
    if (step + j >= n_steps) return true;
    if constexpr (j + 1 < kRing) {
      return self(self, R, step, Slot<j + 1>{});
    } else {
      return false;
    }
  };
  auto walk = [&](auto R) {
    for (int step = 0;; step += kRing)
      if (round(round, R, step, Slot<0>{})) break;
  };

  // zero the slot and P buffer that iteration 0 reads, then start copying
  {
    float* z0 = reinterpret_cast<float*>(ring + (kRing - 1) * TILE);              // Q tile
    float* z1 = reinterpret_cast<float*>(ring + (2 * kRing - 1) * TILE);          // dO tile
    for (int i = tid; i < TILE / 4; i += 512) z0[i] = z1[i] = 0.f;
    float* z2 = reinterpret_cast<float*>(ring + 2 * kRing * TILE + (kRing - 1) * STATS);
    if (tid < STATS / 4) z2[tid] = 0.f;
    float* z3 = reinterpret_cast<float*>(&pshare[1][0]);
    for (int i = tid; i < int(sizeof(pshare[1]) / 4); i += 512) z3[i] = 0.f;
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
#pragma unroll
      for (int e = 0; e < 8; ++e) pprev[qh][0][e] = pprev[qh][1][e] = to_elem<T>(0.f);
  }
  __syncthreads();
  if (dk_role) {
#pragma unroll
    for (int st = 0; st < kAhead; ++st) issue(st);
  }
  if (dk_role)
    walk(std::true_type{});
  else
    walk(std::false_type{});
  __builtin_amdgcn_s_setprio(0);
  wait_copies_barrier<0>();  // no copy in flight when the workgroup ends

  const float mul = dk_role ? a.scale : 1.f;
  if constexpr (RB == 256) {
    // whole-row stores of the wavefront's 32 keys through its 32-row block
    // of the (now idle) rings
    store_block_rows<T, D>(acc, mul, lds_addr(lds) + unsigned(wave) * 32 * RB, [&](int r) {
      const int jk = tile.k0 + kq * 32 + r;
      return jk < tile.k0 + tile.nk
                 ? reinterpret_cast<char*>(dk_role ? a.dk : a.dv) + ((size_t)jk * a.Hkv + g) * RB
                 : nullptr;
    });
  } else if (key_valid) {
    T* op = static_cast<T*>(dk_role ? a.dk : a.dv) + ((size_t)jkey * a.Hkv + g) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        quad t4;
#pragma unroll
        for (int e = 0; e < 4; ++e) t4[e] = to_elem<T>(acc[db][grp * 4 + e] * mul);
        *reinterpret_cast<quad*>(op + db * 32 + grp * 8 + half * 4) = t4;
      }
  }
}

// LDS of the 128-key walk
template <typename T, int D>
constexpr int dkdv_wide_lds_bytes() {
  constexpr int TILE = 64 * D * int(sizeof(T));
  return 2 * 3 * TILE + 3 * 2 * 64 * 4 + 2 * 8 * 128 * int(sizeof(typename Mfma<T>::frag)) + 64 * 4;
}

// One workgroup per CU, taking key tiles until none is left.  16-bit inputs
// walk 128-key tiles and the 64-key remainders of segments (the plan's wide
// list); fp32 walks 64-key tiles.  Both walks share one LDS buffer.
template <typename T, int D>
__global__ __launch_bounds__(512, 1) void tree_attn_dkdv_kernel(BwdArgs a) {
  constexpr int kLds = sizeof(T) == 2 && dkdv_wide_lds_bytes<T, D>() > dkdv_lds_bytes<T, D>()
                           ? dkdv_wide_lds_bytes<T, D>()
                           : dkdv_lds_bytes<T, D>();
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  __shared__ int s_item[2];
  int turn = 0;
  const int n_items = a.n_ktiles * a.Hkv;
  for (int item; (item = take_item(&a.counters[0], n_items, s_item, turn)) >= 0;) {
    int tile_rank, g;
    decode_item(item, a.Hkv, tile_rank, g);
    const KTile tile = a.ktiles[tile_rank];
    if constexpr (sizeof(T) == 2) {
      if (tile.nk > 64)
        dkdv_wide_item<T, D>(a, tile, g, lds);
      else
        dkdv_item<T, D>(a, tile, g, lds);
    } else {
      dkdv_item<T, D>(a, tile, g, lds);
    }
  }
  finish_block(&a.counters[0]);
}

// ---------------------------------------------------------------------------
// 3. dQ, query-major (same walk as the forward kernel)

constexpr int kDqRing = 4;

template <typename T, int D, int HG>
__device__ __forceinline__ void dq_item(const BwdArgs& a, int item) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  using quad = typename M::quad;
  constexpr int BN = 64;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int RB = D * int(sizeof(T));  // bytes of one head's row
  constexpr int TILE = BN * RB;           // bytes of one 64-row tile
  constexpr int kAhead = kDqRing - 1;
  static_assert(RB == 128 || RB == 256, "128- or 256-byte rows");
  static_assert(8 % HG == 0, "eight wavefronts per workgroup");
  static_assert(kDqRing == 4, "the walk is unrolled over four ring slots");

  // K ring then V ring (each 64 KB, so a slot offset fits an LDS immediate)
  __shared__ __attribute__((aligned(16))) char ring[2 * kDqRing * TILE];

  int tile_rank, group;
  decode_item(item, a.Hq / HG, tile_rank, group);
  const QTile tile = a.qtiles[tile_rank];

  // (opaque per item, so nothing derived from the thread index is hoisted
  // out of the item loop to stay live across items)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int col = lane & 31, half = lane >> 5;
  const int ts = wave / HG;
  const int h = group * HG + wave % HG;
  const int g = h / a.G;
  const int qrow = ts * 32 + col;
  const int qtok = tile.q0 + min(qrow, tile.nq - 1);
  const int qpos = tile.pos0 + qrow;
  const int wave_pos0 = tile.pos0 + ts * 32;
  const int kv_len = tile.pos0 + tile.nq;
  const int n_steps = (kv_len + BN - 1) / BN;
  const float c = a.scale * kLog2e;

  frag qf[KS], of[KS];
  {
    const size_t off = ((size_t)qtok * a.Hq + h) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = load_frag<T>(static_cast<const T*>(a.q) + off + ks * 16);
      of[ks] = load_frag<T>(static_cast<const T*>(a.dout) + off + ks * 16);
    }
  }
  const float nlse2 = a.delta[(size_t)a.Hq * a.T + (size_t)h * a.T + qtok];
  const float ndlt = a.delta[(size_t)h * a.T + qtok];

  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = f32x16{};
  f32x16 ndlt16;  // -delta of this lane's query in all 16 entries (set once the loads are in)

  // (per-lane copy offsets: this walk has no vector registers to spare)
  PathCopier<T, RB, false> copier(static_cast<const T*>(a.k), static_cast<const T*>(a.v), g, a.Hkv,
                                  lds_addr(ring), lds_addr(ring + kDqRing * TILE),
                                  a.spans, tile, kv_len, wave, lane);
  auto issue = [&](int step) {
    copier.issue(min(step, n_steps - 1) * BN, (unsigned)(step % kDqRing) * TILE);
  };

  TileAddr<T, D> ka, va;  // per-lane read addresses in slot 0 of each ring
  ka.init(lds_addr(ring), lane);
  va.init(lds_addr(ring + kDqRing * TILE), lane);

  // The two 32-key halves one after the other (only one half's S and dP
  // are live at a time), with half 0's dQ products issued after half 1's S
  // and dP products: half 1's vector work (P, dS) then issues between
  // those independent products while the matrix core works through them.
  // Every accumulator sums in the same order as half by half.
  auto compute = [&](int v0, auto B) {
    constexpr int off = decltype(B)::value * TILE;
    const bool need_mask = v0 + BN - 1 > wave_pos0;  // wave-uniform
    // S and dP - delta of half kb (the dP products accumulate onto -delta:
    // this lane's query is the same in all 16 entries)
    auto products = [&](int kb, f32x16& s, f32x16& dp) {
      s = f32x16{};
      dp = ndlt16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        M::mma(s, ka.row(ks, off + kb * 32 * RB), qf[ks]);
        M::mma(dp, va.row(ks, off + kb * 32 * RB), of[ks]);
      }
    };
    // dS = P (dP - delta) of half kb, P = exp2(S c - lse2)
    auto vector_work = [&](int kb, const f32x16& s, const f32x16& dp, frag (&dsf)[2]) {
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, nlse2));
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (v0 + kb * 32 + c_row(i, half) > qpos) p[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) dsf[i >> 3][i & 7] = to_elem<T>(p[i] * dp[i]);
    };
    auto dq_products = [&](int kb, const frag (&dsf)[2]) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < DB; ++db) M::mma(dq[db], ka.tr(db, off + (kb * 32 + 16 * hh) * RB), dsf[hh]);
    };
    frag ds0[2], ds1[2];
    {
      f32x16 s, dp;
      products(0, s, dp);
      sched_pipeline<kLdsAhead, 2 * KS, frag_reads<T>(false)>();
      vector_work(0, s, dp, ds0);
    }
    {
      f32x16 s, dp;
      products(1, s, dp);
      dq_products(0, ds0);
      vector_work(1, s, dp, ds1);
      if constexpr (frag_reads<T>(false) > 0)
        // (three vector instructions per product slot: measured faster than
        // two, four, six or eight)
        sched_products_then_valu<kLdsAhead, 2 * KS, frag_reads<T>(false), 2 * DB, frag_reads<T>(true), 3>();
    }
    dq_products(1, ds1);
    sched_pipeline<kLdsAhead, 2 * DB, frag_reads<T>(true)>();
  };
  auto body = [&](int step, auto B) {
    // this wave's copies of `step` are done once only the kAhead - 1 newer
    // steps' copies may be in flight; after the barrier every wave's are,
    // and nobody reads the slot refilled next (last read at step - 1)
    wait_copies_barrier<(kAhead - 1) * path_copies(RB)>();
    issue(step + kAhead);
    compute(step * BN, B);
  };

#pragma unroll
  for (int st = 0; st < kAhead; ++st) issue(st);
  // the row loads are waited for only now, after the first copies are issued
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    settle(qf[ks]);
    settle(of[ks]);
  }
  asm volatile("" ::"v"(nlse2), "v"(ndlt));
#pragma unroll
  for (int i = 0; i < 16; ++i) ndlt16[i] = ndlt;
  // unrolled over the ring slots so every LDS offset is a constant
  for (int step = 0;; step += kDqRing) {
    body(step, Slot<0>{});
    if (step + 1 >= n_steps) break;
    body(step + 1, Slot<1>{});
    if (step + 2 >= n_steps) break;
    body(step + 2, Slot<2>{});
    if (step + 3 >= n_steps) break;
    body(step + 3, Slot<3>{});
    if (step + 4 >= n_steps) break;
  }
  wait_copies_barrier<0>();  // no copy in flight when the workgroup ends

  if constexpr (RB == 256) {
    // whole-row stores through this wavefront's 32-row block of the (now
    // idle) ring
    store_block_rows<T, D>(dq, a.scale, lds_addr(ring) + unsigned(wave) * 32 * RB, [&](int r) {
      return ts * 32 + r < tile.nq
                 ? reinterpret_cast<char*>(a.dq) + ((size_t)(tile.q0 + ts * 32 + r) * a.Hq + h) * RB
                 : nullptr;
    });
  } else if (qrow < tile.nq) {
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

// one workgroup per CU, taking items until none is left
template <typename T, int D, int HG>
__global__ __launch_bounds__(512, 1) void tree_attn_dq_kernel(BwdArgs a) {
  __shared__ int s_item[2];
  int turn = 0;
  const int n_items = a.n_qtiles * (a.Hq / HG);
  for (int item; (item = take_item(&a.counters[1], n_items, s_item, turn)) >= 0;) dq_item<T, D, HG>(a, item);
  finish_block(&a.counters[1]);
}

// ---------------------------------------------------------------------------
// launchers (one per stage; tree_attn_bwd runs all three in order)

// Zeroes n consecutive work-item counter blocks: a dK/dV or dQ stage called
// on its own (without the row-statistics stage right before it) starts from
// zeroed counters whatever the workspace held.
__global__ __launch_bounds__(64) void tree_attn_reset_counters_kernel(ItemCounters* __restrict__ c, int n) {
  const int words = n * int(sizeof(ItemCounters) / 4);
  for (int i = threadIdx.x; i < words; i += 64) reinterpret_cast<unsigned*>(c)[i] = 0u;
}

hipError_t launch_reset_counters(ItemCounters* c, int n, hipStream_t stream) {
  hipLaunchKernelGGL(tree_attn_reset_counters_kernel, dim3(1), dim3(64), 0, stream, c, n);
  return hipGetLastError();
}

// one 512-thread workgroup fits a CU (LDS), so the item-taking kernels run
// as many workgroups as the device has CUs (fewer for fewer items)
unsigned persistent_grid(unsigned n_items) {
  static std::atomic<int> cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return n_items;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return n_items;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n_items < unsigned(n) ? n_items : unsigned(n);
}

template <typename T, int D>
hipError_t launch_bwd_rowstat(const BwdArgs& a, hipStream_t stream) {
  constexpr int CPR = D / Chunk<T>::E;
  constexpr int RPB = 256 / CPR;
  // the query run's rows only
  const unsigned rows = (unsigned)(a.q_end - a.q_begin) * (unsigned)a.Hq;
  hipLaunchKernelGGL((tree_attn_rowstat_kernel<T, D>), dim3((rows + RPB - 1) / RPB), dim3(256), 0, stream,
                     static_cast<const T*>(a.out), static_cast<const T*>(a.dout), a.lse, a.delta,
                     a.delta + (size_t)a.Hq * a.T, a.counters, a.T, a.Hq, a.q_begin * a.Hq, a.q_end * a.Hq);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((tree_attn_dkdv_kernel<T, D>), dim3(persistent_grid((unsigned)a.n_ktiles * (unsigned)a.Hkv)),
                     dim3(512), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D, int HG>
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((tree_attn_dq_kernel<T, D, HG>),
                     dim3(persistent_grid((unsigned)a.n_qtiles * (unsigned)(a.Hq / HG))), dim3(512), 0, stream, a);
  return hipGetLastError();
}

template hipError_t launch_bwd_rowstat<__bf16, 128>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_rowstat<__bf16, 64>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_rowstat<float, 64>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dkdv<__bf16, 128>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dkdv<__bf16, 64>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dkdv<float, 64>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<__bf16, 128, 1>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<__bf16, 128, 2>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<__bf16, 128, 4>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<__bf16, 64, 1>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<__bf16, 64, 2>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<__bf16, 64, 4>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<float, 64, 1>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<float, 64, 2>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<float, 64, 4>(const BwdArgs&, hipStream_t);

}  // namespace tree_attn
