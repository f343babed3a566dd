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
// Work decomposition (one workgroup of W wavefronts per compute unit; W = 8,
// or 12 for bf16 rows of 128 with head groups of 4, see below):
//   * a workgroup owns a query tile of 32*NT tokens (inside one segment) and
//     HG query heads of one key/value head (NT*HG = W);
//   * wave w holds 32 query rows (token sub-tile w / HG, head w % HG) with Q
//     in registers;
//   * the workgroup walks the segment's ancestor path as one virtual key
//     sequence (the merged spans of the plan), 64 keys per step.  K and V
//     rows are gathered span by span straight into rings of four LDS tiles
//     (global_load_lds, 16 B per lane, row-major, swizzled), three steps
//     ahead of the compute, with one barrier per step; the loop is unrolled
//     over the ring slots so every LDS read is a per-lane address register
//     plus an immediate offset;
//   * every wave computes S^T = K Q^T (K rows read as A fragments), the
//     online softmax per query column, and O^T += V^T P^T (V read with the
//     transposing LDS load).  A lane owns one query column, so the row max
//     and row sum are in-lane reductions plus one lane swap with lane l ^ 32;
//   * the softmax works in base 2 with the scale folded into one FMA per
//     score, against a reference that is only moved (and O rescaled) when a
//     probability would exceed 2^16; the exponentials are taken against the
//     current reference first and their sum decides whether a step needs the
//     row maximum at all, so most steps compute no maximum.  Numerator and
//     denominator share the reference, so the result is exact;
//   * the own-segment causal rule is "virtual key position <= query
//     position", applied only on the last steps of the walk;
//   * with W = 12 (three wavefronts per SIMD instead of two, so a SIMD has a
//     third instruction stream to issue from while the others wait), each
//     step is taken as two 32-key halves (S, softmax and P V of one half,
//     then of the other), which keeps a wavefront within the 168 registers
//     that three per SIMD leave; waves 0-7 issue the copies, waves 8-11
//     only compute.
#include <type_traits>

#include "kernel_common.hpp"

namespace tree_attn {

// a lane's sum of 32 probabilities above this (2^16) moves the reference
constexpr float kLazyMax = 65536.0f;
constexpr int kFwdRing = 4;

template <int N>
using Slot = std::integral_constant<int, N>;

template <typename T, int D>
constexpr int fwd_ring_bytes() {
  return 2 * kFwdRing * 64 * D * int(sizeof(T));
}

// One work item: query tile `tile_rank` of the plan's list, head group `group`.
template <typename T, int D, int HG, int W>
__device__ __forceinline__ void fwd_item(const FwdArgs& a, int item, char* ring) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  using quad = typename M::quad;
  constexpr int BN = 64;  // keys per step
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int RB = D * int(sizeof(T));  // bytes of one head's row
  constexpr int TILE = BN * RB;           // bytes of one 64-row tile
  constexpr int kAhead = kFwdRing - 1;
  static_assert(RB == 128 || RB == 256, "128- or 256-byte rows");
  static_assert(W == 8 || W == 12, "8 or 12 wavefronts per workgroup");
  static_assert(W % HG == 0, "whole head groups per workgroup");
  constexpr bool kCopier8 = W == 8;  // (else only waves 0-7 issue copies)
  static_assert(kFwdRing == 4, "the walk is unrolled over four ring slots");

  // `ring`: the K ring then the V ring (each 64 KB, so a slot offset fits an
  // LDS immediate)
  int tile_rank, group;
  decode_item(item, a.Hq / HG, tile_rank, group);
  const QTile tile = a.tiles[tile_rank];

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

  // Q: with 12 wavefronts, copied whole-row into ring slots 1-3 (idle until
  // the first steps' copies; K ring for waves 0-5, V ring for waves 6-11)
  // and read from there; else loaded first, its wait coming after the first
  // copies are issued, so both latencies overlap
  constexpr bool kStageQ = W == 12 && RB == 256;
  frag qf[KS];
  unsigned qblk = 0;
  if constexpr (kStageQ) {
    qblk = wave < 6 ? lds_addr(ring) + TILE + unsigned(wave) * 32 * RB
                    : lds_addr(ring + kFwdRing * TILE) + TILE + unsigned(wave - 6) * 32 * RB;
    const char* qb = static_cast<const char*>(a.q) + ((size_t)tile.q0 * a.Hq + h) * RB;
    const unsigned rstride = unsigned(a.Hq) * RB;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = 4 * r + (lane >> 4);
      const unsigned voff = unsigned(min(ts * 32 + row, tile.nq - 1)) * rstride +
                            unsigned(((lane & 15) ^ swz<RB>(row)) * 16);
      copy16_async(qb, voff, qblk + r * 1024);
    }
  } else {
    const T* p = static_cast<const T*>(a.q) + ((size_t)qtok * a.Hq + h) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = load_frag<T>(p + ks * 16);
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  PathCopier<T, RB> copier(static_cast<const T*>(a.k), static_cast<const T*>(a.v), g, a.Hkv, lds_addr(ring),
                           lds_addr(ring + kFwdRing * TILE), a.spans, tile, kv_len, wave,
                           lane);
  // step `step` goes to slot step % kFwdRing; steps past the end re-copy
  // the last step into their (idle) slot so every wave issues the same
  // number of copies per step
  auto issue = [&](int step) {
    if (kCopier8 || wave < 8) copier.issue(min(step, n_steps - 1) * BN, (unsigned)(step % kFwdRing) * TILE);
  };
  TileAddr<T, D> ka, va;  // per-lane read addresses in slot 0 of each ring
  ka.init(lds_addr(ring), lane);
  va.init(lds_addr(ring + kFwdRing * TILE), lane);

  auto compute = [&](int v0, auto B) {
    constexpr int off = decltype(B)::value * TILE;
    f32x16 s[2] = {f32x16{}, f32x16{}};
    // (consecutive products to different accumulators; each sums in the
    // same order)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) M::mma(s[kb], ka.row(ks, off + kb * 32 * RB), qf[ks]);
    sched_pipeline<kLdsAhead, 2 * KS, frag_reads<T>(false)>();

    if (v0 + BN - 1 > wave_pos0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (v0 + kb * 32 + c_row(i, half) > qpos) s[kb][i] = -INFINITY;
    }
    // Probabilities against the current reference m, without a row maximum:
    // a lane whose sum exceeds kLazyMax (a score far above m), or is not a
    // number (the first step, m = -inf), sends the wavefront through the
    // slow path, which moves m to the row maximum, rescales l (O follows
    // right before the P V products) and recomputes.  Every probability of
    // the fast path is at most kLazyMax, so O and l stay far from overflow,
    // and numerator and denominator always share one reference.
    float p[2][16];
    // (the sum starts from the first term, not from an addition to 0)
    float rs;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[kb][i] = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c, -m));
        rs = kb == 0 && i == 0 ? p[0][0] : rs + p[kb][i];
      }
    if (__any(!(rs <= kLazyMax))) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = max_halves(mx) * c;
      const float mnew = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      l *= alpha;
      m = mnew;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[kb][i] = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c, -m));
          rs = kb == 0 && i == 0 ? p[0][0] : rs + p[kb][i];
        }
    }
    l += rs;

    // the denominator sums the fp32 probabilities; only the P*V operand is
    // rounded to the input type
    frag pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) pf[kb][i >> 3][i & 7] = to_elem<T>(p[kb][i]);

#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < DB; ++db) M::mma(o[db], va.tr(db, off + (kb * 32 + 16 * hh) * RB), pf[kb][hh]);
    sched_pipeline<kLdsAhead, 4 * DB, frag_reads<T>(true)>();
  };
  // W = 12: the same step as two 32-key halves (fewer live registers)
  auto compute_halves = [&](int v0, auto B) {
    constexpr int off = decltype(B)::value * TILE;
    const bool diag = v0 + BN - 1 > wave_pos0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) M::mma(s, ka.row(ks, off + kb * 32 * RB), qf[ks]);
      sched_pipeline<kLdsAhead, KS, frag_reads<T>(false)>();
      if (diag) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (v0 + kb * 32 + c_row(i, half) > qpos) s[i] = -INFINITY;
      }
      float p[16];
      // (the sum starts from the first term, not from an addition to 0)
      float rs;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, -m));
        rs = i == 0 ? p[0] : rs + p[i];
      }
      if (__any(!(rs <= kLazyMax))) {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
        mx = max_halves(mx) * c;
        const float mnew = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
        l *= alpha;
        m = mnew;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, -m));
          rs = i == 0 ? p[0] : rs + p[i];
        }
      }
      l += rs;
      frag pf[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) pf[i >> 3][i & 7] = to_elem<T>(p[i]);
      // (consecutive products to different accumulators; each sums in the
      // same order)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < DB; ++db) M::mma(o[db], va.tr(db, off + (kb * 32 + 16 * hh) * RB), pf[hh]);
      sched_pipeline<kLdsAhead, 2 * DB, frag_reads<T>(true)>();
    }
  };
  // A wavefront whose 32 query rows all lie past the tile's end (in the
  // last tile of a segment) copies and waits like the others but computes
  // and stores nothing, so the wavefronts with rows have their SIMD's
  // matrix core to themselves.
  const bool rows_valid = ts * 32 < tile.nq;  // wave-uniform
  auto body = [&](int step, auto B) {
    // this wave's copies of `step` are done once only the kAhead - 1 newer
    // steps' copies may be in flight; after the barrier every wave's are,
    // and nobody reads the slot refilled next (last read at step - 1)
    if (kCopier8 || wave < 8)
      wait_copies_barrier<(kAhead - 1) * path_copies(RB)>();
    else
      wait_copies_barrier<0>();
    issue(step + kAhead);
    if (rows_valid) {
      if constexpr (W == 12)
        compute_halves(step * BN, B);
      else
        compute(step * BN, B);
    }
  };

  if constexpr (kStageQ) {
    // step 0's copies with the Q rows; Q into registers; then steps 1-2
    // into the slots the Q rows leave
    issue(0);
    wait_copies_barrier<0>();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = *reinterpret_cast<const __attribute__((address_space(3))) frag*>(
          (size_t)(qblk + col * RB + (((2 * ks + half) ^ swz<RB>(col)) << 4)));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) settle(qf[ks]);
    wait_copies_barrier<0>();
    issue(1);
    issue(2);
  } else {
#pragma unroll
    for (int st = 0; st < kAhead; ++st) issue(st);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) settle(qf[ks]);
  }
  // unrolled over the ring slots so every LDS offset is a constant
  for (int step = 0;; step += kFwdRing) {
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
  if (!rows_valid) return;

  l = sum_halves(l);
  if constexpr (RB == 256) {
    // whole-row stores through this wavefront's 32-row block of the (now
    // idle) ring
    store_block_rows<T, D>(o, 1.f / l, lds_addr(ring) + unsigned(wave) * 32 * RB, [&](int r) {
      return ts * 32 + r < tile.nq
                 ? reinterpret_cast<char*>(a.out) + ((size_t)(tile.q0 + ts * 32 + r) * a.Hq + h) * RB
                 : nullptr;
    });
    const int ln = lane_now(), col = ln & 31;
    if (ts * 32 + col < tile.nq && ln < 32)
      a.lse[(size_t)h * a.T + tile.q0 + ts * 32 + col] = m * kLn2 + __logf(l);
  } else if (qrow < tile.nq) {
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

// One workgroup per item (work in the plan's longest-first order, spread
// over the XCDs by the dispatcher), or -- with work-item counters from the
// caller's workspace -- one workgroup per CU taking items until none is left
// (the hand-out of the backward walks: XCD-local lists first, then the
// other XCDs' remaining items), which absorbs the XCDs' clock differences.
template <typename T, int D, int HG, bool DYN, int W>
__global__ __launch_bounds__(64 * W, 1) void tree_attn_fwd_kernel(FwdArgs a) {
  // With three wavefronts per SIMD, issue ties go to the oldest, and the
  // youngest third (waves 8-11, which issue no copies) finished each step
  // last while the oldest waited at the barrier; a higher priority for it
  // evens the three out (agent tree -1.4 %).
  if (W == 12 && __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= 8) __builtin_amdgcn_s_setprio(1);
  __shared__ __attribute__((aligned(16))) char ring[fwd_ring_bytes<T, D>()];
  if constexpr (DYN) {
    __shared__ int s_item[2];
    int turn = 0;
    const int n_items = a.n_tiles * (a.Hq / HG);
    for (int item; (item = take_item(a.counters, n_items, s_item, turn)) >= 0;) fwd_item<T, D, HG, W>(a, item, ring);
    finish_block(a.counters);
  } else {
    fwd_item<T, D, HG, W>(a, blockIdx.x, ring);
  }
}

unsigned persistent_grid(unsigned n_items);

// wavefronts per workgroup: 12 for bf16 rows of 128 with head groups of 4
// (96-query tiles), else 8
template <typename T, int D, int HG>
constexpr int fwd_waves() {
  return sizeof(T) == 2 && D == 128 && HG == 4 ? 12 : 8;
}

template <typename T, int D, int HG>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  constexpr int W = fwd_waves<T, D, HG>();
  const unsigned n_items = (unsigned)a.n_tiles * (unsigned)(a.Hq / HG);
  if (a.counters)
    hipLaunchKernelGGL((tree_attn_fwd_kernel<T, D, HG, true, W>), dim3(persistent_grid(n_items)), dim3(64 * W), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((tree_attn_fwd_kernel<T, D, HG, false, W>), dim3(n_items), dim3(64 * W), 0, stream, a);
  return hipGetLastError();
}

// explicit instantiations used by the C ABI
template hipError_t launch_fwd<__bf16, 128, 1>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<__bf16, 128, 2>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<__bf16, 128, 4>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<__bf16, 64, 1>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<__bf16, 64, 2>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<__bf16, 64, 4>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<float, 64, 1>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<float, 64, 2>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<float, 64, 4>(const FwdArgs&, hipStream_t);

}  // namespace tree_attn
