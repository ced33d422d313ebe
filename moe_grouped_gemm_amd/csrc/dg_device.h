// Device code shared by the GEMM kernels (the two FP8 K-loop pipelines
// dg_kernel.hip and dg_kernel_deep.hip, the K-grouped kernel and the FP8 x FP4
// kernel): vector types, the LDS swizzle, waits and barriers, buffer
// descriptors, E8M0 scale codes, the tile scheduler of the M-grouped layouts
// with its on-device group table, and the contiguous layout's row masks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "dg_internal.h"

namespace dg {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) i32x4 global_i32x4;

constexpr int BK = 128;        // K block = scale granularity
constexpr int ROW_BYTES = 128; // one tile row of one K block

// Byte offset of 16-byte chunk `c` (0..7) of tile row `row` in LDS. Rows are
// 128 bytes; chunks are XOR-swizzled with (row / 2) % 8.
//
// gfx950 serves a ds_read_b128 half-wave by half-wave, each half in two
// passes of 16 lanes: lane l goes to pass (bit 2 ^ bit 3 ^ bit 4 of l), and a
// pass takes one LDS cycle when its lanes hit 16 distinct 16-byte bank slots
// (address bits 4..7), one more cycle per extra lane on a slot. With this
// swizzle and the fragment chunk choice of lds_offsets() (lane group
// g = lane / 16 reads chunks g and g + 4) every pass of a fragment read is
// conflict-free: 4 cycles per instruction, where chunks 2g and 2g + 1 take 8.
__device__ __forceinline__ int lds_offset(int row, int c) {
  return row * ROW_BYTES + ((c ^ ((row >> 1) & 7)) << 4);
}

// s_waitcnt through the builtin (not inline asm), so that the compiler's own
// wait insertion knows what has already been waited for. gfx9 encoding:
// vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_vmcnt_0() { wait_vmcnt<0>(); }

// Workgroup barrier without the memory fence that __syncthreads() adds: the
// callers wait on exactly the counters they need first. The empty asm
// statements keep the compiler from moving LDS accesses across it: the
// direct-to-LDS loads write through bare addresses, so to the compiler the
// stage buffers look unchanged by other waves, and the barrier intrinsic
// itself touches no memory.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_lgkmcnt_0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// c + the 16x16 block of products of a and b summed over K = 128, OCP E4M3
// operands without block scales: v_mfma_f32_16x16x128_f8f6f4. The compiler
// exposes the f8f6f4 MFMAs only through the block-scaled builtin, and for
// scale operands that are constant zero it selects this plain instruction
// (no scale registers, checked in the generated code and by a CPU test of
// the build) whose products are not scaled -- a scale code given in a
// register would instead be applied as 2^(code - 127). The integer-exact
// GPU tests, bit for bit against the oracle, pin that the products come out
// unscaled.
__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same with E8M0 block scales: c + 2^(ea - 127) * 2^(eb - 127) * (the
// products of a and b summed over K = 128), ea applied to the first
// operand's row of each lane and eb to the second's.
__device__ __forceinline__ f32x4 mfma_fp8_scaled(const i32x8& a, const i32x8& b, f32x4 c, int ea, int eb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}

// The E8M0 code of a float32 scale: its biased exponent field e, which the
// MFMA's block-scale operand reads as 2^(e - 127) (e = 255: NaN). For a
// positive normal power of two this is the scale itself; sign and mantissa
// bits are ignored.
__device__ __forceinline__ int e8m0_code(float s) {
  return (int)((__builtin_bit_cast(uint32_t, s) >> 23) & 0xFFu);
}

// Where one output tile's operands live, and which of its rows are valid.
struct TileRef {
  const uint8_t* a;    // row 0 of the group's A
  const float* sfa;    // the group's transposed LHS scales
  const uint8_t* b;    // the group's B [n][k]
  const float* sfb;    // the group's RHS scales [n/128][k/128]
  uint16_t* d;         // row 0 of the group's D
  int group;
  int m0, n0;          // first row (within the group) and column of the tile
  int load_rows;       // A rows at or beyond this are not loaded (they read as zero)
  int valid_rows;      // dense / masked: rows below this are written
  bool active;         // false: no such tile (past the end, or nothing to compute)
};

// Raw buffer descriptor (gfx9 word 3: 32-bit data format). Loads at byte
// offsets at or beyond `bytes` return zero without touching memory.
// The caller guarantees that base and bytes are the same in every lane; they
// are moved to scalar registers so that the descriptor is scalar.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// The LDS destination of a direct-to-LDS load, given as a bare LDS byte
// address: the compiler then does not associate the load with an LDS variable
// and adds no waits of its own before later LDS accesses (it cannot tell
// which parts of a variable a load in flight writes, and would wait for every
// load in flight before reading or writing any of it). Every access to loaded
// data is ordered after its load explicitly: a vmcnt wait, then a barrier.
__device__ __forceinline__ lds_void* lds_dest(uint32_t lds_addr) {
  return (lds_void*)(uintptr_t)__builtin_amdgcn_readfirstlane(lds_addr);
}

// Maps a linear tile index to (m block, n block), walking panels of
// `panel_m` consecutive M blocks across all N blocks so that tiles issued
// together share A and B panels in L2.
__device__ __forceinline__ void raster(int t, int m_blocks, int n_blocks, int panel_m, int& mb, int& nb) {
  const int per_panel = panel_m * n_blocks;
  const int panel = t / per_panel;
  const int r = t - panel * per_panel;
  const int rows_here = min(panel_m, m_blocks - panel * panel_m);
  mb = panel * panel_m + r % rows_here;
  nb = r / rows_here;
}

// aux[i] for a wave-uniform i, read through the scalar cache: a scalar load,
// so reading it never waits for this wave's outstanding vector memory
// operations (refills and stores in flight).
__device__ __forceinline__ int aux_scalar(const int* aux, int i) {
  typedef const __attribute__((address_space(4))) int* const_i32_ptr;
  const uint64_t v = reinterpret_cast<uint64_t>(aux);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  const const_i32_ptr base = (const_i32_ptr)((static_cast<uint64_t>(hi) << 32) | lo);
  return base[__builtin_amdgcn_readfirstlane(i)];
}

// The group table of the layouts whose row counts are read on the device
// (masked, no-padding), built by wave 0 at kernel start from the counts in
// aux, 64 groups at a time with an in-wave scan:
//   tab[g], g = 0..G:          tiles of the groups before g (each group: its
//                              BM-row blocks times the N blocks);
//   tab[G + 1 + g], g = 0..G:  no-padding only: first row of group g. The
//                              groups' rows follow one another from row 0;
//                              whatever lies at or past row m is cut off.
// A count is clamped to [0, m] (masked: m is max_m). Returns the table once
// every wave of the workgroup can read it.
template <class C, int KIND>
__device__ int* group_table(const GemmArgs& p, int tid) {
  static_assert(counts_on_device(KIND), "masked and no-padding layouts only");
  __shared__ int tab[GROUP_TABLE_INTS];
  const int G = p.num_groups;
  if (tid < 64) {
    const int lane = tid;
    int tiles_before = 0;
    long long rows_before = 0;
    for (int g0 = 0; g0 < G; g0 += 64) {
      const int g = g0 + lane;
      const int rows = g < G ? min(max(p.aux[g], 0), p.m) : 0;
      long long rows_incl = rows;
      for (int d = 1; d < 64; d <<= 1) {
        const long long v = __shfl_up(rows_incl, d);
        if (lane >= d) rows_incl += v;
      }
      int first = 0, count = rows;
      if constexpr (KIND == KIND_NOPAD) {
        const long long s = rows_before + rows_incl - rows;
        first = (int)min(s, (long long)p.m);
        count = (int)min(s + rows, (long long)p.m) - first;
      }
      const int tiles = (count + C::BM - 1) / C::BM * p.n_blocks;
      int tiles_incl = tiles;
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(tiles_incl, d);
        if (lane >= d) tiles_incl += v;
      }
      if (g < G) {
        tab[g] = tiles_before + tiles_incl - tiles;
        if constexpr (KIND == KIND_NOPAD) tab[G + 1 + g] = first;
      }
      tiles_before += __shfl(tiles_incl, 63);
      rows_before += __shfl(rows_incl, 63);
    }
    if (lane == 0) {
      tab[G] = tiles_before;
      if constexpr (KIND == KIND_NOPAD) tab[2 * G + 1] = (int)min(rows_before, (long long)p.m);
    }
  }
  __syncthreads();
  return tab;
}

// Resolves linear tile index t of layout KIND. Tile order:
//   dense:      raster over (M block, N block);
//   contiguous: slot-major, then raster over (BM-row block, N block); slot j
//               of a block is the j-th distinct valid group among its 128-row
//               segment blocks (a block holds two groups only where a group's
//               segment ends inside it), so slot 0 carries nearly all work;
//   masked,
//   no-padding: per group (the group table, built on the device from the
//               per-group row counts), then N block, then M block.
template <class C, int KIND>
__device__ __forceinline__ TileRef resolve_tile(const GemmArgs& p, int t, int num_tiles, const int* s_prefix) {
  TileRef tr;
  tr.active = false;
  if (t >= num_tiles) return tr;
  const size_t K = (size_t)p.k;
  const int k_blocks = p.k / BK;
  if constexpr (counts_on_device(KIND)) {
    int lo = 0, hi = p.num_groups - 1;  // last g with prefix[g] <= t: a group with tiles
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_prefix[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    int v;
    if constexpr (KIND == KIND_NOPAD) {
      // The group's rows: a row range of the shared A, sfa and D.
      const int first = s_prefix[p.num_groups + 1 + g];
      v = s_prefix[p.num_groups + 2 + g] - first;
      tr.a = p.a + (size_t)first * K;
      tr.sfa = p.sfa + first;
      tr.d = p.d + (size_t)first * p.n;
    } else {
      // The group's own [max_m] slice of A, sfa and D.
      v = min(max(aux_scalar(p.aux, g), 0), p.m);
      tr.a = p.a + (size_t)g * p.m * K;
      tr.sfa = p.sfa + (size_t)g * k_blocks * p.ld_sfa;
      tr.d = p.d + (size_t)g * p.m * p.n;
    }
    const int mblocks = (v + C::BM - 1) / C::BM;
    const int local = t - s_prefix[g];
    const int nb = local / mblocks;
    const int mb = local - nb * mblocks;
    tr.group = g;
    tr.b = p.b + (size_t)g * p.n * K;
    tr.sfb = p.sfb + (size_t)g * (p.n / BK) * k_blocks;
    tr.m0 = mb * C::BM;
    tr.n0 = nb * C::BN;
    tr.load_rows = v;        // rows past the group's count are never fetched
    tr.valid_rows = v;
    tr.active = true;
  } else {
    const int per_slot = p.m_blocks * p.n_blocks;
    const int slot = t / per_slot;
    int mb, nb;
    raster(t - slot * per_slot, p.m_blocks, p.n_blocks, 4, mb, nb);
    tr.m0 = mb * C::BM;
    tr.n0 = nb * C::BN;
    tr.load_rows = p.m;
    tr.valid_rows = p.m;
    tr.a = p.a;
    tr.sfa = p.sfa;
    tr.d = p.d;
    tr.group = 0;
    tr.b = p.b;
    tr.sfb = p.sfb;
    if constexpr (KIND == KIND_CONTIGUOUS) {
      // The distinct valid groups of this block's 128-row segment blocks, in order.
      int found = 0, g_sel = -1;
#pragma unroll
      for (int j = 0; j < C::SLOTS; ++j) {
        const int r = tr.m0 + 128 * j;
        const int g = r < p.m ? aux_scalar(p.aux, r) : -1;
        bool fresh = g >= 0 && g < p.num_groups;
#pragma unroll
        for (int i = 0; i < j; ++i) {
          const int ri = tr.m0 + 128 * i;
          if (ri < p.m && aux_scalar(p.aux, ri) == g) fresh = false;
        }
        if (fresh) {
          if (found == slot) g_sel = g;
          ++found;
        }
      }
      if (g_sel < 0) return tr;  // nothing for this slot: inactive
      tr.group = g_sel;
      tr.b = p.b + (size_t)g_sel * p.n * K;
      tr.sfb = p.sfb + (size_t)g_sel * (p.n / BK) * k_blocks;
    }
    tr.active = true;
  }
  return tr;
}

__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// The first active tile at or after t in this CTA's sequence t, t+grid, ...
// Every field is the same in all lanes; it is moved to scalar registers.
template <class C, int KIND>
__device__ __forceinline__ TileRef next_active(const GemmArgs& p, int& t, int grid, int num_tiles,
                                               const int* s_prefix) {
  for (; t < num_tiles; t += grid) {
    TileRef tr = resolve_tile<C, KIND>(p, t, num_tiles, s_prefix);
    if (tr.active) {
      tr.a = uniform_ptr(tr.a);
      tr.sfa = uniform_ptr(tr.sfa);
      tr.b = uniform_ptr(tr.b);
      tr.sfb = uniform_ptr(tr.sfb);
      tr.d = uniform_ptr(tr.d);
      tr.group = uniform_int(tr.group);
      tr.m0 = uniform_int(tr.m0);
      tr.n0 = uniform_int(tr.n0);
      tr.load_rows = uniform_int(tr.load_rows);
      tr.valid_rows = uniform_int(tr.valid_rows);
      return tr;
    }
  }
  TileRef none;
  none.active = false;
  return none;
}

// Contiguous layout: which of a wave's 128 tile rows are computed for the
// tile's group. Lane l loads the group indices of rows wm0 + 2l and wm0 + 2l + 1 of
// a tile one tile ahead of use (RowGroups); the K loop turns them into bit
// masks (RowMask: bit l of `even` / `odd` is row 2l / 2l + 1) at a point
// where the loads have landed long before, so that waiting for them does
// not wait for the refills in flight.
struct RowGroups {
  int even, odd;
};
struct RowMask {
  uint64_t even, odd;
};

template <class C>
__device__ __forceinline__ RowGroups load_row_groups(const GemmArgs& p, const TileRef& tr, int wm0, int lane) {
  static_assert(C::WM == 128, "a wave's tile rows are exactly one 128-row block of the layout");
  RowGroups rg{-1, -1};
  const int r = tr.m0 + wm0 + 2 * lane;
  if (tr.active && r < p.m) rg.even = p.aux[r];
  if (tr.active && r + 1 < p.m) rg.odd = p.aux[r + 1];
  return rg;
}

// The contiguous layout's row rule: a 128-row block belongs to the group
// named by its first row's id, and a row of it is computed for that group
// when the row's own id is the same (segments are aligned to 128 rows, so
// in a well-formed layout every valid row passes). A wave's 128 rows are one
// such block and lane 0's `even` row is its first row.
__device__ __forceinline__ RowMask row_mask(const RowGroups& rg, int group) {
  const bool block_is_group = __builtin_amdgcn_readlane(rg.even, 0) == group;
  return RowMask{__builtin_amdgcn_ballot_w64(block_is_group && rg.even == group),
                 __builtin_amdgcn_ballot_w64(block_is_group && rg.odd == group)};
}

// Bits 0..7 of x moved to the even bit positions 0..14.
__device__ __forceinline__ uint32_t spread8(uint32_t x) {
  x = (x | (x << 4)) & 0x0F0Fu;
  x = (x | (x << 2)) & 0x3333u;
  return (x | (x << 1)) & 0x5555u;
}

// Wave-uniform mask of the valid rows of band mt (bit R: tile row
// wm0 + 16 mt + R): from the row mask in the contiguous layout, else the rows
// below the tile's valid-row count.
template <class C, int KIND>
__device__ __forceinline__ uint32_t band_rows(const TileRef& tr, const RowMask& cm, int wm0, int mt) {
  if constexpr (KIND == KIND_CONTIGUOUS) {
    const uint32_t e = (uint32_t)(cm.even >> (8 * mt)) & 0xFFu;
    const uint32_t o = (uint32_t)(cm.odd >> (8 * mt)) & 0xFFu;
    return spread8(e) | (spread8(o) << 1);
  } else {
    const int n = min(max(tr.valid_rows - (tr.m0 + wm0 + 16 * mt), 0), 16);
    return (1u << n) - 1u;
  }
}

}  // namespace dg
