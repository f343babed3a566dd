// Shared device-side building blocks of the gfx950 tree-attention kernels.
//
// Matrix-core conventions (CDNA3/CDNA4 32x32 MFMA):
//   * A operand: lane l supplies row (l % 32) of a 32 x K block;
//   * B operand: lane l supplies column (l % 32) of a K x 32 block;
//   * A and B lanes hold the same K-slot set per register element, so any
//     consistent assignment of reduction indices to (lane half, element) works;
//   * C/D: lane l holds column (l % 32) and rows 8*(i/4) + 4*(l/32) + (i%4),
//     i = 0..15.
// Every contraction here is written so that the C layout of one product is
// directly the B operand of the next: a lane keeps one query (or one key)
// column, and its 16 values are the rows 8*(i/4) + 4*half + (i%4).  A B
// fragment of 8 values i in [8c, 8c+8) therefore covers rows
// {16c + 4*half + 0..3} and {16c + 8 + 4*half + 0..3}; the matching A
// fragment reads those two 4-element runs from a transposed LDS tile.
//
// bf16 tensors use v_mfma_f32_32x32x16_bf16 (one instruction per 16-deep
// step); fp32 tensors use eight v_mfma_f32_32x32x2_f32, which keeps full fp32
// products and accumulation.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.hpp"

namespace tree_attn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
  using frag = bf16x8;  // 8 elements: one 16-deep step of a 32x32 product
  using quad = bf16x4;
  __device__ static inline void mma(f32x16& c, const frag& a, const frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag cat(const quad& lo, const quad& hi) {
    return frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
};

template <>
struct Mfma<float> {
  using frag = f32x8;
  using quad = f32x4;
  __device__ static inline void mma(f32x16& c, const frag& a, const frag& b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
  }
  __device__ static inline frag cat(const quad& lo, const quad& hi) {
    return frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
};

// 16-byte chunk of a tensor row (8 bf16 or 4 fp32 elements).
template <typename T>
struct Chunk {
  static constexpr int E = 16 / int(sizeof(T));
  u32x4 bits;
  __device__ inline T elem(int e) const {
    const T* p = reinterpret_cast<const T*>(&bits);
    return p[e];
  }
};

template <typename T>
__device__ inline Chunk<T> load_chunk(const T* p) {
  Chunk<T> c;
  c.bits = *reinterpret_cast<const u32x4*>(p);
  return c;
}

template <typename T>
__device__ inline Chunk<T> zero_chunk() {
  Chunk<T> c;
  c.bits = u32x4{0u, 0u, 0u, 0u};
  return c;
}

template <typename T>
__device__ inline void store_chunk(T* p, const Chunk<T>& c) {
  *reinterpret_cast<u32x4*>(p) = c.bits;
}

// 8 consecutive elements as an MFMA fragment (16 B for bf16, 32 B for fp32).
template <typename T>
__device__ inline typename Mfma<T>::frag load_frag(const T* p) {
  return *reinterpret_cast<const typename Mfma<T>::frag*>(p);
}

// ---------------------------------------------------------------------------
// LDS tiles: 64 rows (tokens) of RB = D * sizeof(T) bytes (one head's row:
// 256 B for bf16 D = 128 and fp32 D = 64, 128 B for bf16 D = 64), stored
// row-major with the 16-byte chunks of row r XOR-swizzled by swz<RB>(r).
// With 64 banks x 4 B (256 bytes per cycle) both read patterns are free of
// bank conflicts:
//   * row reads (ds_read_b128, 16 lanes per cycle) touch 16 consecutive rows
//     (aligned) at one logical chunk;
//   * transposing reads (ds_read_b64_tr_b16, 32 lanes per cycle) touch 4
//     consecutive rows (aligned) x 4 consecutive chunks (aligned).
// RB = 256 (16 chunks, one row per 256-byte bank line): f(r) = ((r&3)<<2) |
//   ((r>>2)&3) takes all 16 values on 16 aligned rows; on 4 aligned rows x 4
//   aligned chunks, chunk 4m + x and f = 4y + k give 4(m^y) + (x^k), 16
//   distinct chunks.
// RB = 128 (8 chunks, rows r and r+1 share a bank line, in its two halves):
//   with t = (r>>1) & 7, f(r) = t ^ ((t&1)<<2) is a permutation of 0..7 in t,
//   so 16 aligned rows hit 2 x 8 distinct half-lines; of 4 aligned rows, the
//   two of each parity have t of different parity, hence f differing in bit 2,
//   so their 4-chunk runs land in opposite halves of the 8 chunks.
// Both swizzles repeat every 16 rows, so a 16-row block offset is a plain
// byte offset.  Tiles are filled with global_load_lds_dwordx4: lane l of a
// wave writes the 16 bytes at (wave base + 16 l), so each lane loads the
// global chunk that belongs at that swizzled position.

template <int RB>
__device__ inline int swz(int row) {
  static_assert(RB == 128 || RB == 256, "128- or 256-byte rows");
  if constexpr (RB == 256) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    const int t = (row >> 1) & 7;
    return t ^ ((t & 1) << 2);
  }
}

typedef __attribute__((address_space(3))) void lds_void;

// Copies global -> LDS written as inline assembly, for kernels that keep
// several copies in flight and count them themselves.  The compiler does not
// see these as LDS writes, so it adds no wait of its own before LDS reads
// (with the builtin it sometimes waits for every copy in flight); the caller
// orders them with wait_copies_barrier<N>().  Lane l reads
// sbase + voff(l) (sbase wave-uniform) and writes LDS byte address
// lds + size * l (lds wave-uniform).  Nothing else in such a kernel may
// rely on M0 (no dynamic register indexing, no builtin LDS copies).  (The
// LDS address goes through readfirstlane: the compiler may hold a uniform
// value in a vector register, which the scalar operand cannot take.)
__device__ inline void copy16_async(const void* sbase, unsigned voff, unsigned lds) {
  const unsigned m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m)
               : "memory");
}
__device__ inline void copy4_async(const void* sbase, unsigned voff, unsigned lds) {
  const unsigned m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(m)
               : "memory");
}

// LDS byte address of a __shared__ object.
__device__ inline unsigned lds_addr(const void* p) { return (unsigned)(size_t)(const lds_void*)p; }

// An empty asm use of `f`: the compiler completes the loads that produce it
// here, not at its first real use (inside a loop, that wait would also
// drain the copies in flight).  Wider than 16 bytes it goes element-wise.
template <typename F>
__device__ inline void settle(const F& f) {
  if constexpr (sizeof(F) == 16) {
    asm volatile("" ::"v"(f));
  } else {
#pragma unroll
    for (int j = 0; j < int(sizeof(F) / 4); ++j) asm volatile("" ::"v"(f[j]));
  }
}

// Waits until at most N of this wave's vector-memory operations are in
// flight and its LDS operations are done, then joins the workgroup barrier.
// Loads complete in issue order, so with N = the copies issued after a given
// step's, that step's copies (from every wave) are in LDS after the barrier.
template <int N>
__device__ inline void wait_copies_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Software pipelining of LDS fragment reads against the products that use
// them.  After N products, each fed by an A fragment read from LDS, this
// asks the scheduler for: AHEAD fragments' reads, then (one product, one
// fragment's reads) repeated, then the last AHEAD products -- so reads run
// AHEAD fragments in front of the matrix cores instead of each read waiting
// right before its product.  READS = LDS instructions per fragment (bf16:
// one ds_read_b128 per row fragment, two ds_read_b64_tr_b16 per transposed
// one; fp32 needs more and is not pipelined).
constexpr int kLdsAhead = 3;
constexpr int kSchedMfma = 0x0008;
constexpr int kSchedDsRead = 0x0100;

template <typename T>
constexpr int frag_reads(bool transposed) {
  return sizeof(T) == 2 ? (transposed ? 2 : 1) : 0;
}

template <int AHEAD, int N, int READS>
__device__ inline void sched_pipeline() {
  if constexpr (READS > 0 && N > AHEAD) {
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, AHEAD * READS, 0);
#pragma unroll
    for (int i = 0; i < N - AHEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, READS, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, AHEAD, 0);
  }
}

// Per-lane LDS byte addresses of the fragments a wavefront reads from a
// 64-row tile (layout of tile_off), kept in registers for the whole kernel.
// A read adds a compile-time byte offset (ring slot, tile, row block that is
// a multiple of 16 rows) which the LDS instruction takes as an immediate;
// the swizzle repeats every 16 rows, so the per-lane part does not depend
// on the row block.  The addresses are made opaque to the compiler so it
// keeps exactly these registers instead of re-deriving one per offset.
//   row(ks):  the A/B fragment of row (block + lane % 32), elements
//             [16 ks + 8 half, +8);
//   tr(db):   the transposed A fragment of columns [32 db, +32): lane l gets
//             column 32 db + l % 32 and the 8 rows {block + 4h + 0..3} and
//             {block + 8 + 4h + 0..3}, h = l / 32 -- the rows a C-layout B
//             fragment covers (see the header comment).  bf16 uses two
//             ds_read_b64_tr_b16: within each 16-lane group, lane i receives
//             element i % 4 of the 8-byte pieces read by lanes 4j + i / 4
//             (j = 0..3), so lane 4j + k of group g reads row
//             block + 4 (g / 2) + j at column 32 db + 16 (g % 2) + 4 k.
//             fp32 reads the same elements one by one.
template <typename T, int D>
struct TileAddr;

template <int D>
struct TileAddr<__bf16, D> {
  static constexpr int KS = D / 16, DB = D / 32, RB = 2 * D;
  using frag = Mfma<__bf16>::frag;
  unsigned rowa[KS];
  unsigned tra[DB][2];

  __device__ void init(unsigned tile, int lane) {
    const int col = lane & 31, half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      rowa[ks] = tile + col * RB + (((2 * ks + half) ^ swz<RB>(col)) * 16);
      asm volatile("" : "+v"(rowa[ks]));
    }
    const int g = lane >> 4, k = lane & 15;
    const int rr = 4 * (g >> 1) + (k >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = db * 32 + 16 * (g & 1) + 4 * (k & 3);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int row = rr + 8 * p;
        tra[db][p] = tile + row * RB + (((d >> 3) ^ swz<RB>(row)) * 16) + (d & 7) * 2;
        asm volatile("" : "+v"(tra[db][p]));
      }
    }
  }
  __device__ inline frag row(int ks, int off) const {
    return *reinterpret_cast<const __attribute__((address_space(3))) frag*>((size_t)(rowa[ks] + off));
  }
  __device__ inline frag tr(int db, int off) const {
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) s16x4*>((size_t)(tra[db][0] + off)));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) s16x4*>((size_t)(tra[db][1] + off)));
    return Mfma<__bf16>::cat(__builtin_bit_cast(bf16x4, a), __builtin_bit_cast(bf16x4, b));
  }
};

template <int D>
struct TileAddr<float, D> {
  static constexpr int KS = D / 16, DB = D / 32, RB = 4 * D;
  using frag = Mfma<float>::frag;
  unsigned rowa[KS][2];
  unsigned tra[DB][8];

  __device__ void init(unsigned tile, int lane) {
    const int col = lane & 31, half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        rowa[ks][j] = tile + col * RB + (((4 * ks + 2 * half + j) ^ swz<RB>(col)) * 16);
        asm volatile("" : "+v"(rowa[ks][j]));
      }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = db * 32 + col;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = 8 * (j >> 2) + 4 * half + (j & 3);
        tra[db][j] = tile + row * RB + (((d >> 2) ^ swz<RB>(row)) * 16) + (d & 3) * 4;
        asm volatile("" : "+v"(tra[db][j]));
      }
    }
  }
  __device__ inline frag row(int ks, int off) const {
    const f32x4 lo = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>((size_t)(rowa[ks][0] + off));
    const f32x4 hi = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>((size_t)(rowa[ks][1] + off));
    return frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ inline frag tr(int db, int off) const {
    frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      f[j] = *reinterpret_cast<const __attribute__((address_space(3))) float*>((size_t)(tra[db][j] + off));
    return f;
  }
};

// As sched_pipeline over two groups of products in order, N1 products of
// READS1 LDS reads each and then N2 of READS2 (the reads run AHEAD products
// ahead across the boundary), with up to VALU vector instructions after
// each product of the second group (and VALU1 after each of the first):
// vector work of the same wavefront that needs only earlier results then
// issues while the matrix core works through the products.
constexpr int kSchedValu = 0x0002;

template <int AHEAD, int N1, int READS1, int N2, int READS2, int VALU, int VALU1 = 0>
__device__ inline void sched_products_then_valu() {
  static_assert(READS1 > 0 && READS2 > 0 && N1 > AHEAD && N2 > AHEAD, "LDS-fed products");
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, AHEAD * READS1, 0);
#pragma unroll
  for (int i = 0; i < N1 + N2; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    const int next = i + AHEAD;  // the product whose operands are read now
    if (next < N1)
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, READS1, 0);
    else if (next < N1 + N2)
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, READS2, 0);
    if (i >= N1)
      __builtin_amdgcn_sched_group_barrier(kSchedValu, VALU, 0);
    else if (VALU1 > 0)
      __builtin_amdgcn_sched_group_barrier(kSchedValu, VALU1, 0);
  }
}

// Combine v over lanes l and l ^ 32 (the two halves of a wavefront) with one
// VALU lane swap instead of an LDS permute: v_permlane32_swap with both
// operands v returns v's lanes 0..31 twice and its lanes 32..63 twice.
__device__ inline float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row offset of C-layout value i for lane half `half`.
__device__ inline constexpr int c_row(int i, int half) { return 8 * (i >> 2) + 4 * half + (i & 3); }

template <typename T>
__device__ inline T to_elem(float x) {
  return T(x);
}

// This lane's index in its wavefront, computed where it is used: an opaque
// instruction pair, so values derived from it are not computed ahead of a
// loop and held in registers through it.
__device__ inline int lane_now() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Writes a wavefront's 32 x D block, held in the C layout (lane l: block row
// l % 32; acc[db][i]: column 32 db + c_row(i, l / 32)), times `mul`, to 32
// global rows of RB = 256 bytes, through a 32-row LDS block `blk` (byte
// address; free, and read by no other wavefront), so that every store
// writes whole rows.  Straight from the C layout each store instruction
// would put 8 or 16 bytes into each of 32 rows a head-row apart: 32 partial
// cache lines.  The block is swizzled like the tiles (two-way bank
// conflicts on the writes, none on the row reads).  `row_ptr(r)` is the
// global address of block row r; rows with row_ptr(r) == nullptr are
// skipped.
template <typename T, int D, class RowPtr>
__device__ inline void store_block_rows(const f32x16 (&acc)[D / 32], float mul, unsigned blk, RowPtr row_ptr) {
  constexpr int RB = D * int(sizeof(T));
  static_assert(RB == 256, "256-byte rows");
  using quad = typename Mfma<T>::quad;
  const int ln = lane_now();
  const int col = ln & 31, half = ln >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      quad t4;
#pragma unroll
      for (int e = 0; e < 4; ++e) t4[e] = to_elem<T>(acc[db][grp * 4 + e] * mul);
      const int byte = (db * 32 + grp * 8 + half * 4) * int(sizeof(T));
      const unsigned at = blk + col * RB + (((byte >> 4) ^ swz<RB>(col)) << 4) + (byte & 15);
      *reinterpret_cast<__attribute__((address_space(3))) quad*>((size_t)at) = t4;
    }
  const int r16 = ln >> 4, ch = ln & 15;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = 4 * j + r16;
    const u32x4 v4 = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
        (size_t)(blk + row * RB + ((ch ^ swz<RB>(row)) << 4)));
    char* p = reinterpret_cast<char*>(row_ptr(row));
    if (p) *reinterpret_cast<u32x4*>(p + ch * 16) = v4;
  }
}

// Work-item decode.  Workgroups are dispatched round-robin over the 8 XCDs
// (each with its own L2), so block b runs on XCD b % 8.  When the head
// groups split evenly over the XCDs, each XCD gets a contiguous range of
// head groups (all query heads of one key/value head land on one XCD and
// share its L2) and walks its tiles longest-first.
__device__ inline void decode_item(int b, int n_groups, int& tile_rank, int& group) {
  if (n_groups % 8 == 0) {
    const int xcd = b & 7, k = b >> 3, gper = n_groups >> 3;
    group = xcd * gper + k % gper;
    tile_rank = k / gper;
  } else {
    tile_rank = b / n_groups;
    group = b % n_groups;
  }
}

// Dynamic hand-out of work items across the XCDs.  Under these kernels the
// eight XCDs of one GPU run at clocks up to ~5 % apart, so a split of the
// items by block index alone leaves the slowest XCD finishing last.  Here the
// grid is one workgroup per CU, and each workgroup takes items until none is
// left: first from the ticket counter of the XCD it runs on -- that XCD's
// share of the static split (items b with b % 8 == xcd, in order: longest
// first, with XCD-local head groups) -- and once that list is exhausted,
// from the other XCDs' lists (their remaining, shortest items).  A pass over
// the eight lists that finds nothing means every item has been taken (the
// lists only shrink).  The last workgroup to finish zeroes the counters for
// the next launch (the first launch on a new workspace relies on the
// row-statistics stage having zeroed them).
struct ItemCounters {
  unsigned next[8];
  unsigned done;
  unsigned pad[7];
};

// the next item for this workgroup, or -1 when none is left (ends with a
// barrier: the previous item is finished by every wave).  The item is passed
// through one of two LDS words, alternating between calls (`turn` is the
// caller's, flipped here): a wave may still be reading one call's word while
// thread 0 writes the next call's, and the word comes round again only after
// a barrier that every wave reaches once it has read it.
__device__ inline int take_item(ItemCounters* ctr, int n_items, int (&s_item)[2], int& turn) {
  turn ^= 1;
  if (threadIdx.x == 0) {
    unsigned xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    int item = -1;
    for (unsigned k = 0; k < 8; ++k) {
      const unsigned x = (xcc + k) & 7u;
      const unsigned t = atomicAdd(&ctr->next[x], 1u);
      if ((long long)t * 8 + x < n_items) {
        item = int(t * 8 + x);
        break;
      }
    }
    s_item[turn] = item;
  }
  __syncthreads();
  return s_item[turn];
}

__device__ inline void finish_block(ItemCounters* ctr) {
  if (threadIdx.x == 0 && atomicAdd(&ctr->done, 1u) == gridDim.x - 1) {
#pragma unroll
    for (int x = 0; x < 8; ++x) __hip_atomic_store(&ctr->next[x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&ctr->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One span record through the scalar data cache: the address is
// wave-uniform, the result lands in scalar registers, and the load is waited
// for inside the same asm block (lgkmcnt counts scalar loads and LDS
// operations, not the global->LDS copies, so it never waits behind those).
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ inline Span load_span(const Span* p) {
  i32x4 r;
  asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(p) : "memory");
  return Span{r[0], r[1], r[2], r[3]};
}

// Copies of a segment's ancestor path, as one virtual key sequence, into
// LDS rings for the 512-thread query-major kernels.  Step `step` covers the
// 64 virtual positions [64 step, 64 step + 64); its K rows go to a 64-row
// tile of the K ring and its V rows to the same slot of the V ring
// (row-major, swizzled).  Waves 0-3 copy K rows, waves 4-7 V rows, 16 rows
// each; one copy instruction moves 1 KB = 1024 / RB rows, so every wave
// issues exactly path_copies(RB) copies per step.  The first span record
// comes with the query tile's record; later ones are read from the plan in
// global memory with scalar loads, one at a time, so a path may have any
// number of spans and nothing is staged before the walk.
// A step inside one span (the common case: spans are usually much longer
// than 64) takes its rows from one base; otherwise the wave visits the spans
// the step overlaps in order and each lane takes its row from the one that
// holds it.  Positions past the path read the last valid row (the caller
// masks them).  Byte offsets of rows must fit in 32 bits (checked by the
// host).  With SCALAR_BASE, in the one-span case the step's first row goes
// into the wave-uniform base address (scalar arithmetic) and each lane adds
// a fixed offset computed once, so the copies cost no vector instructions
// (four more vector registers held for the offsets).
__host__ __device__ constexpr int path_copies(int RB) { return 16 * RB / 1024; }

template <typename T, int RB, bool SCALAR_BASE = true>
struct PathCopier {
  static constexpr int NC = path_copies(RB);  // copies per wave per step
  static constexpr int RPC = 1024 / RB;       // rows per copy
  static constexpr int LPR = RB / 16;         // lanes per row
  const T* base;       // K (waves 0-3) or V (waves 4-7) of this key/value head
  unsigned row_bytes;  // bytes between consecutive tokens
  unsigned lds;        // this wave's first row in slot 0 of its ring
  unsigned chunk[NC];  // this lane's swizzled byte offset in its row, per copy
  unsigned lane_off[NC];  // (row + RPC r) * row_bytes + chunk[r]: the one-span case's per-lane offset
  int row;             // this lane's row of copy 0 (copy r: row + RPC r)
  const Span* spans;   // the segment's spans (global memory)
  int ucur;            // wave-uniform span cursor
  int cphys, clen, cvirt;  // spans[ucur], kept in scalar registers
  int kv_len;          // positions on the path

  // spans: the plan's span list; tile: the query tile whose ancestor path
  // is walked (it names the path's first span and holds a copy of it)
  __device__ PathCopier(const T* k, const T* v, int g, int Hkv, unsigned k_ring, unsigned v_ring,
                        const Span* all_spans, const QTile& tile, int len, int wave, int lane) {
    base = (wave < 4 ? k : v) + (size_t)g * RB / sizeof(T);
    row_bytes = (unsigned)Hkv * RB;
    const int r0 = (wave & 3) * 16;
    lds = (wave < 4 ? k_ring : v_ring) + r0 * RB;
    row = r0 + lane / LPR;
#pragma unroll
    for (int r = 0; r < NC; ++r) {
      chunk[r] = unsigned(((lane % LPR) ^ swz<RB>(row + RPC * r)) * 16);
      if constexpr (SCALAR_BASE) lane_off[r] = unsigned(row + RPC * r) * row_bytes + chunk[r];
    }
    spans = all_spans + tile.span0;
    ucur = 0;
    kv_len = len;
    cphys = tile.phys0;
    clen = tile.len0;
    cvirt = tile.virt0;
  }

  // positions [v0, v0 + 64) into the ring slot at byte offset `slot`
  __device__ inline void issue(int v0, unsigned slot) {
    // the current span stays in scalar registers: a step inside it (the
    // common case) loads nothing
    while (v0 >= cvirt + clen) {
      const Span sp = load_span(spans + (++ucur));
      cphys = sp.phys;
      clen = sp.len;
      cvirt = sp.virt;
    }
    const bool one_span = v0 + 64 <= cvirt + clen && v0 + 64 <= kv_len;
    if (SCALAR_BASE && one_span) {
      const char* sb = reinterpret_cast<const char*>(base) + size_t(unsigned(cphys + (v0 - cvirt))) * row_bytes;
#pragma unroll
      for (int r = 0; r < NC; ++r) copy16_async(sb, lane_off[r], lds + slot + RPC * r * RB);
    } else {
      int phys[NC];
      if (one_span) {
#pragma unroll
        for (int r = 0; r < NC; ++r) phys[r] = cphys + (v0 - cvirt) + row + RPC * r;
      } else {
        // the spans the step overlaps, from the current one (which holds v0)
        int v[NC];
#pragma unroll
        for (int r = 0; r < NC; ++r) {
          v[r] = min(v0 + row + RPC * r, kv_len - 1);
          phys[r] = 0;
        }
        const int hi = min(v0 + 63, kv_len - 1);  // the last position of the step
        int k = ucur, sphys = cphys, slen = clen, svirt = cvirt;
        for (;;) {
#pragma unroll
          for (int r = 0; r < NC; ++r)
            if (v[r] >= svirt && v[r] < svirt + slen) phys[r] = sphys + (v[r] - svirt);
          if (svirt + slen > hi) break;
          const Span sp = load_span(spans + (++k));
          sphys = sp.phys;
          slen = sp.len;
          svirt = sp.virt;
        }
      }
#pragma unroll
      for (int r = 0; r < NC; ++r)
        copy16_async(base, (unsigned)phys[r] * row_bytes + chunk[r], lds + slot + RPC * r * RB);
    }
  }
};

struct FwdArgs {
  ItemCounters* counters;  // work-item hand-out (caller workspace), or null: one workgroup per item
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const QTile* tiles;
  const Span* spans;
  int32_t n_tiles;
  int32_t T, Hq, Hkv, G;
  float scale;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;
  ItemCounters* counters;  // [0]: dK/dV pass, [1]: dQ pass (in the workspace)
  const QTile* qtiles;
  const KTile* ktiles;
  const Span* spans;
  int32_t n_qtiles, n_ktiles;
  int32_t T, Hq, Hkv, G;
  int32_t q_begin, q_end;  // the plan's query run
  float scale;
};

}  // namespace tree_attn
