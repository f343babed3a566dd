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

// Two 4-element runs p[0..3] and p[8..11] as one fragment (transposed tiles).
template <typename T>
__device__ inline typename Mfma<T>::frag load_frag_split(const T* p) {
  using quad = typename Mfma<T>::quad;
  return Mfma<T>::cat(*reinterpret_cast<const quad*>(p), *reinterpret_cast<const quad*>(p + 8));
}

// ---------------------------------------------------------------------------
// LDS tiles: ROWS x D elements, one 256-byte row per token, stored row-major
// with the 16 16-byte chunks of row r XOR-swizzled by
// f(r) = ((r&3)<<2) | ((r>>2)&3).  With 64 banks x 4 B (256 bytes per cycle)
// both read patterns are free of bank conflicts:
//   * row reads (ds_read_b128, 16 lanes per cycle): 16 consecutive rows
//     (aligned) at one logical chunk land on 16 distinct chunks, since f takes
//     all 16 values there;
//   * transposing reads (ds_read_b64_tr_b16, 32 lanes per cycle): 4
//     consecutive rows (aligned) x 4 consecutive chunks (aligned): with
//     chunk = 4m + x and f = 4y + k the physical chunk is 4(m^y) + (x^k), 16
//     distinct values.
// Tiles are filled with global_load_lds_dwordx4: lane l of a wave writes the
// 16 bytes at (wave base + 16 l), so each lane loads the global chunk that
// belongs at that swizzled position.

constexpr int kRowBytes = 256;
constexpr int kChunksPerRow = kRowBytes / 16;

__device__ inline int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// element offset of logical chunk `chunk` of `row` in a tile of element type T
template <typename T>
__device__ inline int tile_off(int row, int chunk) {
  return row * (kRowBytes / int(sizeof(T))) + ((chunk ^ swz(row)) * (16 / int(sizeof(T))));
}

typedef __attribute__((address_space(3))) void lds_void;

// Asynchronous 16-byte-per-lane copy global -> LDS (wave-uniform LDS base).
__device__ inline void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_base, 16, 0, 0);
}

__device__ inline void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Copies global -> LDS written as inline assembly, for kernels that keep
// several copies in flight and count them themselves.  The compiler does not
// see these as LDS writes, so it adds no wait of its own before LDS reads
// (with the builtin it sometimes waits for every copy in flight); the caller
// orders them with wait_copies_barrier<N>().  Lane l reads
// sbase + voff(l) (sbase wave-uniform) and writes LDS byte address
// lds + size * l (lds wave-uniform).  Nothing else in such a kernel may
// rely on M0 (no dynamic register indexing, no builtin LDS copies).
__device__ inline void copy16_async(const void* sbase, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory");
}
__device__ inline void copy4_async(const void* sbase, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
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

// Fragment of 8 consecutive elements [e0, e0+8) of a tile row (e0 % 8 == 0).
template <typename T>
__device__ inline typename Mfma<T>::frag tile_row_frag(const T* tile, int row, int e0) {
  constexpr int E = 16 / int(sizeof(T));
  if constexpr (E == 8) {
    return *reinterpret_cast<const typename Mfma<T>::frag*>(tile + tile_off<T>(row, e0 / E));
  } else {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(tile + tile_off<T>(row, e0 / E));
    const f32x4 hi = *reinterpret_cast<const f32x4*>(tile + tile_off<T>(row, e0 / E + 1));
    return typename Mfma<T>::frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Transposed A fragment: lane l gets column d = d0 + (l % 32) of the tile and
// the 8 rows {r0 + 4h + 0..3} and {r0 + 8 + 4h + 0..3}, h = l / 32 -- the
// rows a C-layout B fragment covers (see the header comment).  bf16 uses two
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i%4
// of the 8-byte pieces read by lanes 4j + i/4 (j = 0..3), so lane 4j+k of
// group g reads row r0 + 4(g/2) + j at column d0 + 16(g%2) + 4k.  fp32 reads
// the same elements one by one.
template <typename T>
__device__ inline typename Mfma<T>::frag tile_tr_frag(const T* tile, int r0, int d0, int lane) {
  if constexpr (sizeof(T) == 2) {
    const int g = lane >> 4, k = lane & 15;
    const int row = r0 + 4 * (g >> 1) + (k >> 2);
    const int d = d0 + 16 * (g & 1) + 4 * (k & 3);
    const T* p0 = tile + tile_off<T>(row, d >> 3) + (d & 7);
    const T* p1 = tile + tile_off<T>(row + 8, d >> 3) + (d & 7);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p0);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p1);
    const bf16x4 lo = __builtin_bit_cast(bf16x4, a);
    const bf16x4 hi = __builtin_bit_cast(bf16x4, b);
    return Mfma<T>::cat(lo, hi);
  } else {
    const int h = lane >> 5, d = d0 + (lane & 31);
    typename Mfma<T>::frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = r0 + 8 * (j >> 2) + 4 * h + (j & 3);
      f[j] = tile[tile_off<T>(row, d >> 2) + (d & 3)];
    }
    return f;
  }
}

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
//             [16 ks + 8 half, +8) -- tile_row_frag;
//   tr(db):   the transposed fragment of rows (block + 0..15) and columns
//             [32 db, +32) -- tile_tr_frag.
template <typename T, int D>
struct TileAddr;

template <int D>
struct TileAddr<__bf16, D> {
  static constexpr int KS = D / 16, DB = D / 32;
  using frag = Mfma<__bf16>::frag;
  unsigned rowa[KS];
  unsigned tra[DB][2];

  __device__ void init(unsigned tile, int lane) {
    const int col = lane & 31, half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      rowa[ks] = tile + col * kRowBytes + (((2 * ks + half) ^ swz(col)) * 16);
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
        tra[db][p] = tile + row * kRowBytes + (((d >> 3) ^ swz(row)) * 16) + (d & 7) * 2;
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
  static constexpr int KS = D / 16, DB = D / 32;
  using frag = Mfma<float>::frag;
  unsigned rowa[KS][2];
  unsigned tra[DB][8];

  __device__ void init(unsigned tile, int lane) {
    const int col = lane & 31, half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        rowa[ks][j] = tile + col * kRowBytes + (((4 * ks + 2 * half + j) ^ swz(col)) * 16);
        asm volatile("" : "+v"(rowa[ks][j]));
      }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = db * 32 + col;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = 8 * (j >> 2) + 4 * half + (j & 3);
        tra[db][j] = tile + row * kRowBytes + (((d >> 2) ^ swz(row)) * 16) + (d & 3) * 4;
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

// As sched_pipeline, and VALU instructions after every matrix product, so
// that independent vector work of the same wavefront runs while the matrix
// core is busy.
constexpr int kSchedValu = 0x0002;

template <int AHEAD, int N, int READS, int VALU>
__device__ inline void sched_pipeline_valu() {
  if constexpr (READS > 0 && N > AHEAD) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, AHEAD * READS, 0);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if (READS > 0 && i < N - AHEAD) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, READS, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedValu, VALU, 0);
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

// A segment's merged spans are staged in LDS once per workgroup, so span
// lookups use the LDS counter and never wait behind in-flight global->LDS
// copies.  A segment may have at most kMaxSpans spans (checked by the host).
constexpr int kMaxSpans = 256;

// Copies the spans of segment `seg` to LDS (every thread takes part; the
// caller synchronises before use).
__device__ inline void stage_spans(Span* lds_spans, const int32_t* span_ptr, const Span* spans, int seg) {
  const int first = span_ptr[seg], n = span_ptr[seg + 1] - first;
  for (int i = threadIdx.x; i < n; i += blockDim.x) lds_spans[i] = spans[first + i];
}

// Monotone cursor over a segment's merged spans: maps a virtual key position
// of the reconstructed sequence to its physical token.
struct SpanCursor {
  const Span* spans;  // LDS copy
  int cur;
  __device__ inline int phys(int v) {
    while (v >= spans[cur].virt + spans[cur].len) ++cur;
    return spans[cur].phys + (v - spans[cur].virt);
  }
};

// Copies of a segment's ancestor path, as one virtual key sequence, into
// LDS rings for the 512-thread query-major kernels.  Step `step` covers the
// 64 virtual positions [64 step, 64 step + 64); its K rows go to a 64-row
// tile of the K ring and its V rows to the same slot of the V ring
// (row-major, swizzled).  Waves 0-3 copy K rows, waves 4-7 V rows, 16 rows
// each in 4 instructions, so every wave issues exactly kPathCopies copies
// per step.  A step inside one span (the common case: spans are usually
// much longer than 64) takes its rows from one base; otherwise each lane
// looks its rows up with a per-lane span cursor.  Positions past the path
// read the last valid row (the caller masks them).  Byte offsets of rows
// must fit in 32 bits (checked by the host).
constexpr int kPathCopies = 4;

template <typename T>
struct PathCopier {
  const T* base;       // K (waves 0-3) or V (waves 4-7) of this key/value head
  unsigned row_bytes;  // bytes between consecutive tokens
  unsigned lds;        // this wave's first row in slot 0 of its ring
  unsigned chunk[4];   // this lane's swizzled byte offset in its row, per copy
  int row;             // this lane's row of copy 0 (copy r: row + 4 r)
  const Span* spans;   // the segment's spans, in LDS
  int ucur, lcur;      // wave-uniform and per-lane span cursors
  int kv_len;          // positions on the path

  __device__ PathCopier(const T* k, const T* v, int g, int Hkv, unsigned k_ring, unsigned v_ring, const Span* sp,
                        int len, int wave, int lane) {
    base = (wave < 4 ? k : v) + (size_t)g * kRowBytes / sizeof(T);
    row_bytes = (unsigned)Hkv * kRowBytes;
    const int r0 = (wave & 3) * 16;
    lds = (wave < 4 ? k_ring : v_ring) + r0 * kRowBytes;
    row = r0 + (lane >> 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) chunk[r] = unsigned(((lane & 15) ^ swz(row + 4 * r)) * 16);
    spans = sp;
    ucur = 0;
    lcur = 0;
    kv_len = len;
  }

  // positions [v0, v0 + 64) into the ring slot at byte offset `slot`
  __device__ inline void issue(int v0, unsigned slot) {
    while (v0 >= spans[ucur].virt + spans[ucur].len) ++ucur;
    const Span sp = spans[ucur];
    int phys[4];
    if (v0 + 64 <= sp.virt + sp.len && v0 + 64 <= kv_len) {
#pragma unroll
      for (int r = 0; r < 4; ++r) phys[r] = sp.phys + (v0 - sp.virt) + row + 4 * r;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = min(v0 + row + 4 * r, kv_len - 1);
        while (v >= spans[lcur].virt + spans[lcur].len) ++lcur;
        phys[r] = spans[lcur].phys + (v - spans[lcur].virt);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      copy16_async(base, (unsigned)phys[r] * row_bytes + chunk[r], lds + slot + 4 * r * kRowBytes);
  }
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const QTile* tiles;
  const int32_t* span_ptr;
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
  const QTile* qtiles;
  const KTile* ktiles;
  const int32_t* span_ptr;
  const Span* spans;
  int32_t n_qtiles, n_ktiles;
  int32_t T, Hq, Hkv, G;
  float scale;
};

}  // namespace tree_attn
