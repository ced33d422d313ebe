// FP8 (OCP E4M3) NT GEMM with 1x128 LHS / 128x128 RHS float32 scales and BF16
// output, dense and M-grouped (contiguous, masked), for gfx950 (MI355X).
//
// One persistent kernel serves the three layouts ("DeepGEMM for PPU" README,
// "Optimizations": one block scheduler for the non-grouped and grouped
// kernels, rasterised for L2 reuse). Per output tile and per 128-wide K block:
//
//   1. HBM -> LDS: the A tile [BM][128] and B tile [BN][128] bytes and the
//      tile's LHS scales, with 16-byte direct-to-LDS loads
//      (global_load_lds_dwordx4), STAGES deep;
//   2. matrix cores: one v_mfma_f32_16x16x128_f8f6f4 per 16x16 sub-tile gives
//      the block's float32 partial sum;
//   3. promotion: total += partial * (sfa[m] * sfb[n/128]) in float32
//      ("Persistent warp-specialization": promotion overlapped with data
//      movement and MMA);
//   4. after the last K block, BF16 round-to-nearest-even and store of the
//      rows that are valid for the layout.
//
// The MFMA is issued with the B fragment as its first operand and the A
// fragment as its second, so that each lane's four results share one output
// row m (lane % 16) and four consecutive columns: one LHS scale per lane per
// 16-row band, and an 8-byte store per lane per sub-tile.

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

constexpr int BK = 128;        // K block = scale granularity
constexpr int ROW_BYTES = 128; // one tile row of one K block

// Byte offset of 16-byte chunk `c` (0..7) of tile row `row` in LDS. Rows are
// 128 bytes; chunks are XOR-swizzled with (row / 2) % 8 so that the 16 rows
// read by one 16-lane group of a ds_read_b128 fall on all 64 banks once.
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
// callers wait on exactly the counters they need first.
__device__ __forceinline__ void barrier() { __builtin_amdgcn_s_barrier(); }
__device__ __forceinline__ void wait_lgkmcnt_0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// One LDS buffer per pipeline stage, each its own variable: the compiler can
// then tell a direct-to-LDS load into one stage from reads of another and
// does not wait for the in-flight stage before reading the current one.
template <class C, int S>
__device__ __forceinline__ uint8_t* stage_buf() {
  static_assert(S < C::STAGES, "stage index");
  __shared__ __attribute__((aligned(1024))) uint8_t buf[C::STAGE_BYTES];
  return buf;
}

// One 16-byte direct-to-LDS load per lane; the LDS destination of lane l is
// lds_base + 16 * l (lds_base must be the same for the whole wave).
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_base, 16, 0, 0);
}
// One 4-byte direct-to-LDS load per lane; destination lds_base + 4 * l.
__device__ __forceinline__ void dma4(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_base, 4, 0, 0);
}

// 32 bytes (logical chunks 2*(lane/16) and 2*(lane/16)+1) of tile row `row`:
// the MFMA operand of one lane for one 128-wide K block. The same lane ->
// K mapping is used for both operands, so the products pair the same k.
__device__ __forceinline__ i32x8 read_frag(const uint8_t* tile, int row, int lane) {
  const int c0 = (lane >> 4) << 1;
  const i32x4 x = *reinterpret_cast<const i32x4*>(tile + lds_offset(row, c0));
  const i32x4 y = *reinterpret_cast<const i32x4*>(tile + lds_offset(row, c0 + 1));
  return (i32x8){x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

// Read-only global memory seen through the constant address space: a load
// at a wave-uniform address through such a pointer is a scalar load.
typedef const __attribute__((address_space(4))) float* const_f32_ptr;

// A pointer the compiler cannot prove wave-uniform, moved to scalar registers
// (the caller guarantees it is uniform) and typed as read-only.
__device__ __forceinline__ const_f32_ptr uniform_const_ptr(const float* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return (const_f32_ptr)((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
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

// One wave-wide 16-byte buffer load per lane into LDS: lane l writes
// lds_base + 16 * l (lds_base is the same for the whole wave).
__device__ __forceinline__ void buf_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void buf_dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 4, voff, 0, 0, 0);
}

// Per-lane byte offsets of this lane's loads within a tile, fixed for the
// kernel: row * K + 16 * chunk for the A and B tile loads (the j-th load of a
// wave adds j * NW * 8 rows), and 4 * row for the scale load.
struct LaneOffsets {
  uint32_t ab;
  uint32_t ab_step;    // bytes between a wave's consecutive tile loads
  uint32_t sa;
};

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

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_>
struct Config {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, STAGES = STAGES_;
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int THREADS = NW * 64;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int MT = WM / 16, NT = WN / 16;
  static constexpr int SLOTS = BM / 128;  // contiguous layout: 128-row segment blocks per tile row block
  static constexpr int A_DMA = BM * ROW_BYTES / 1024 / NW;  // 1 KB per wave-wide 16-byte load
  static constexpr int B_DMA = BN * ROW_BYTES / 1024 / NW;
  // LHS scales: wave w loads rows [w * SA_ROWS, w * SA_ROWS + 64) of the tile
  // into its own 256-byte region; row r is read from region r / SA_ROWS.
  static constexpr int SA_ROWS = BM / NW;
  // Per stage and wave: A and B tile loads, one scale load, the RHS scale.
  static constexpr int LOADS_PER_STAGE = A_DMA + B_DMA + 1 + 1;
  static constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
  static constexpr int SA_BYTES = NW * 256;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SA_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static_assert(BM % 128 == 0, "tile rows are whole 128-row blocks");
  static_assert(BM % (WAVES_M * 16) == 0 && BN % (WAVES_N * 16) == 0, "wave tile");
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns lie in one 128-column scale block");
  static_assert(BM * ROW_BYTES % (1024 * NW) == 0 && BN * ROW_BYTES % (1024 * NW) == 0, "DMA split");
  static_assert(SA_ROWS <= 64 && BM % NW == 0, "scale load granularity");
};

// Resolves linear tile index t of layout KIND. Tile order:
//   dense:      raster over (M block, N block);
//   contiguous: slot-major, then raster over (BM-row block, N block); slot j
//               of a block is the j-th distinct valid group among its 128-row
//               segment blocks (a block holds two groups only where a group's
//               segment ends inside it), so slot 0 carries nearly all work;
//   masked:     per group (prefix sums of the per-group tile counts, read
//               from masked_m on the device), then N block, then M block.
template <class C, int KIND>
__device__ __forceinline__ TileRef resolve_tile(const GemmArgs& p, int t, int num_tiles, const int* s_prefix) {
  TileRef tr;
  tr.active = false;
  if (t >= num_tiles) return tr;
  const size_t K = (size_t)p.k;
  const int k_blocks = p.k / BK;
  if constexpr (KIND == KIND_MASKED) {
    int lo = 0, hi = p.num_groups - 1;  // last g with prefix[g] <= t: a group with tiles
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_prefix[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int v = min(max(p.aux[g], 0), p.m);
    const int mblocks = (v + C::BM - 1) / C::BM;
    const int local = t - s_prefix[g];
    const int nb = local / mblocks;
    const int mb = local - nb * mblocks;
    tr.group = g;
    tr.a = p.a + (size_t)g * p.m * K;
    tr.sfa = p.sfa + (size_t)g * k_blocks * p.ld_sfa;
    tr.b = p.b + (size_t)g * p.n * K;
    tr.sfb = p.sfb + (size_t)g * (p.n / BK) * k_blocks;
    tr.d = p.d + (size_t)g * p.m * p.n;
    tr.m0 = mb * C::BM;
    tr.n0 = nb * C::BN;
    tr.load_rows = v;        // rows past masked_m are never fetched
    tr.valid_rows = v;
    tr.active = true;
  } else {
    const int per_slot = p.m_blocks * p.n_blocks;
    const int slot = t / per_slot;
    int mb, nb;
    raster(t - slot * per_slot, p.m_blocks, p.n_blocks, 8, mb, nb);
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
        const int g = r < p.m ? p.aux[r] : -1;
        bool fresh = g >= 0 && g < p.num_groups;
#pragma unroll
        for (int i = 0; i < j; ++i) {
          const int ri = tr.m0 + 128 * i;
          if (ri < p.m && p.aux[ri] == g) fresh = false;
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

template <class C>
__device__ __forceinline__ LaneOffsets lane_offsets(int k, int wave, int lane) {
  LaneOffsets o;
  const int row0 = wave * 8 + (lane >> 3);
  const int c = (lane & 7) ^ ((row0 >> 1) & 7);  // the same for every load of the wave (NW * 8 % 16 == 0)
  o.ab = (uint32_t)row0 * (uint32_t)k + (uint32_t)c * 16u;
  o.ab_step = (uint32_t)(C::NW * 8) * (uint32_t)k;
  o.sa = (uint32_t)(wave * C::SA_ROWS + lane) * 4u;
  return o;
}

// Buffer descriptors of K block `kb` of one tile.
struct StageSrc {
  __amdgpu_buffer_rsrc_t a, b, sa, sb;
  uint32_t sb_off;
};

template <class C>
__device__ __forceinline__ StageSrc stage_src(const TileRef& tr, int kb, const GemmArgs& p, int wn0) {
  StageSrc r;
  const uint32_t K = (uint32_t)p.k;
  const int k_blocks = p.k / BK;
  const uint32_t a_rows = (uint32_t)min(max(tr.load_rows - tr.m0, 0), C::BM);
  const uint32_t b_rows = (uint32_t)min(p.n - tr.n0, C::BN);
  r.a = buffer_rsrc(tr.a + (size_t)tr.m0 * K + (size_t)kb * BK, a_rows * K);
  r.b = buffer_rsrc(tr.b + (size_t)tr.n0 * K + (size_t)kb * BK, b_rows * K);
  r.sa = buffer_rsrc(tr.sfa + (size_t)kb * p.ld_sfa + tr.m0, a_rows * 4u);
  const float* sfb_row = tr.sfb + (size_t)((min(tr.n0 + wn0, p.n - 1)) / BK) * k_blocks;
  r.sb = buffer_rsrc(sfb_row, (uint32_t)k_blocks * 4u);
  r.sb_off = (uint32_t)kb * 4u;
  return r;
}

// The loads of one K block into stage S are issued in STAGE_PARTS parts
// spread over the first bands of the current K step, so that the memory
// pipeline drains while the matrix cores work: part 0 and 1 the A tile (rows
// past the tile's valid rows read as zero), part 2 and 3 the B tile (both with
// the swizzle of lds_offset()), part 3 also the tile's LHS scales and the RHS
// scale of this wave's columns (returned; usable once the stage has been
// waited for).
constexpr int STAGE_PARTS = 4;

template <class C, int S, int PART>
__device__ __forceinline__ float issue_part(const StageSrc& r, int wave, const LaneOffsets& lo) {
  static_assert(C::A_DMA % 2 == 0 && C::B_DMA % 2 == 0, "loads split in halves");
  uint8_t* st = stage_buf<C, S>();
  if constexpr (PART < 2) {
#pragma unroll
    for (int j = PART * C::A_DMA / 2; j < (PART + 1) * C::A_DMA / 2; ++j)
      buf_dma16(r.a, lo.ab + j * lo.ab_step, st + (j * C::NW + wave) * 1024);
    return 0.f;
  } else {
#pragma unroll
    for (int j = (PART - 2) * C::B_DMA / 2; j < (PART - 1) * C::B_DMA / 2; ++j)
      buf_dma16(r.b, lo.ab + j * lo.ab_step, st + C::A_BYTES + (j * C::NW + wave) * 1024);
    if constexpr (PART == 3) {
      buf_dma4(r.sa, lo.sa, st + C::A_BYTES + C::B_BYTES + wave * 256);
      const uint32_t bits = __builtin_amdgcn_raw_buffer_load_b32(r.sb, r.sb_off, 0, 0);
      return __builtin_bit_cast(float, bits);
    }
    return 0.f;
  }
}

template <class C, int S>
__device__ __forceinline__ float issue_stage(const TileRef& tr, int kb, const GemmArgs& p, int wave, int wn0,
                                             const LaneOffsets& lo) {
  const StageSrc r = stage_src<C>(tr, kb, p, wn0);
  issue_part<C, S, 0>(r, wave, lo);
  issue_part<C, S, 1>(r, wave, lo);
  issue_part<C, S, 2>(r, wave, lo);
  return issue_part<C, S, 3>(r, wave, lo);
}

// Wait until this wave's loads of the stage about to be read have landed,
// when `ahead` later stages' loads may still be in flight.
template <class C>
__device__ __forceinline__ void wait_stage(int ahead) {
  if constexpr (C::STAGES >= 4) {
    if (ahead >= 2) { wait_vmcnt<2 * C::LOADS_PER_STAGE>(); return; }
  }
  if constexpr (C::STAGES >= 3) {
    if (ahead >= 1) { wait_vmcnt<C::LOADS_PER_STAGE>(); return; }
  }
  wait_vmcnt_0();
}

// Position of tile row r's LHS scale in a stage's scale area.
template <class C>
__device__ __forceinline__ int sa_index(int r) {
  return (r / C::SA_ROWS) * 64 + r % C::SA_ROWS;
}

// Per-wave state of the tile being computed.
template <class C>
struct WaveTile {
  f32x4 acc[C::MT][C::NT];
  bool row_ok[C::MT];
  bool on;  // the wave has a valid row and valid columns: it runs its MFMAs and stores
};

// The K loop of one tile, with global K steps counted from stage PHASE. Each
// step waits for its stage, refills the stage freed by the previous step with
// the block STAGES-1 steps ahead (from the next tile once this one runs out),
// and computes one 128-wide K block.
template <class C, int KIND, int PHASE>
__device__ __forceinline__ void mainloop(const GemmArgs& p, const TileRef& cur, const TileRef& nxt,
                                         WaveTile<C>& wt, float& sb_next, int wave, int wm0, int wn0, int lane,
                                         const LaneOffsets& lo) {
  const int k_blocks = p.k / BK;
  for (int kb0 = 0; kb0 < k_blocks; kb0 += C::STAGES) {
    static_for<0, C::STAGES>([&](auto si) {
      constexpr int step = decltype(si)::value;
      constexpr int s = (step + PHASE) % C::STAGES;
      const int kb = kb0 + step;
      if (kb >= k_blocks) return;
      wait_stage<C>(C::STAGES - 2);
      wait_lgkmcnt_0();
      barrier();
      // Refill the stage every wave finished reading in the previous step.
      // Past the end of this tile the loads belong to the next one; with no
      // next tile the last block is loaded again (nobody reads it): the
      // loads are issued unconditionally, since a branch here would make the
      // compiler wait for them before reading the current stage.
      constexpr int sr = (s + C::STAGES - 1) % C::STAGES;
      const int ahead = kb + C::STAGES - 1;
      const bool own = ahead < k_blocks;
      const TileRef& src = (own || !nxt.active) ? cur : nxt;
      const int kb_load = own ? ahead : (nxt.active ? ahead - k_blocks : k_blocks - 1);
      const StageSrc rsrc = stage_src<C>(src, kb_load, p, wn0);
      const float sb = sb_next;  // this step's RHS scale, loaded with its stage
      if (!wt.on) {
        issue_part<C, sr, 0>(rsrc, wave, lo);
        issue_part<C, sr, 1>(rsrc, wave, lo);
        issue_part<C, sr, 2>(rsrc, wave, lo);
        sb_next = issue_part<C, sr, 3>(rsrc, wave, lo);
        return;
      }

      const uint8_t* As = stage_buf<C, s>();
      const uint8_t* Bs = As + C::A_BYTES;
      const float* SAs = reinterpret_cast<const float*>(As + C::A_BYTES + C::B_BYTES);

      // Pipeline over the wave's 16-row bands: the next band's A fragment and
      // scale are read while this band's MFMAs run; each band's partial sums
      // are promoted right after its MFMAs (the other wave on the SIMD keeps
      // the matrix core busy meanwhile); the first bands also issue the
      // refill loads.
      i32x8 bf[C::NT];
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) bf[nt] = read_frag(Bs, wn0 + nt * 16 + (lane & 15), lane);
      i32x8 af = read_frag(As, wm0 + (lane & 15), lane);
      float sa = SAs[sa_index<C>(wm0 + (lane & 15))];
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
        i32x8 af_next;
        float sa_next = 0.f;
        if (mt + 1 < C::MT) {
          af_next = read_frag(As, wm0 + (mt + 1) * 16 + (lane & 15), lane);
          sa_next = SAs[sa_index<C>(wm0 + (mt + 1) * 16 + (lane & 15))];
        }
        if (mt == 0) issue_part<C, sr, 0>(rsrc, wave, lo);
        if (mt == 1) issue_part<C, sr, 1>(rsrc, wave, lo);
        if (mt == 2) issue_part<C, sr, 2>(rsrc, wave, lo);
        if (mt == 3) sb_next = issue_part<C, sr, 3>(rsrc, wave, lo);
        f32x4 part[C::NT];
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt)
          part[nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[nt], af, (f32x4){0.f, 0.f, 0.f, 0.f}, 0,
                                                                     0, 0, 0, 0, 0);
        const float w = sa * sb;
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) wt.acc[mt][nt] += part[nt] * w;
        if (mt + 1 < C::MT) {
          af = af_next;
          sa = sa_next;
        }
        // Issue order: the next band's reads and this band's share of the
        // refill first, then the MFMAs, then the promotion of this band.
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // DS reads
        if (mt < STAGE_PARTS) __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);  // VMEM loads
        __builtin_amdgcn_sched_group_barrier(0x008, C::NT, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4 * C::NT + 1, 0);  // VALU
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  }
}

template <class C, int KIND>
__global__ void __launch_bounds__(C::THREADS, 1) fp8_gemm_nt_kernel(GemmArgs p) {
  static_assert(C::STAGES == 2, "the cross-tile refill assumes one stage in flight");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar scale loads
  const int wave_m = wave / C::WAVES_N;
  const int wave_n = wave % C::WAVES_N;
  const int wm0 = wave_m * C::WM;
  const int wn0 = wave_n * C::WN;
  const int k_blocks = p.k / BK;

  // Per-group tile counts for the masked layout, read on the device.
  int num_tiles = p.num_tiles;
  [[maybe_unused]] int* s_prefix = nullptr;
  if constexpr (KIND == KIND_MASKED) {
    __shared__ int prefix[MAX_MASKED_GROUPS + 1];
    s_prefix = prefix;
    if (tid == 0) {
      int acc = 0;
      for (int g = 0; g < p.num_groups; ++g) {
        s_prefix[g] = acc;
        const int v = min(max(p.aux[g], 0), p.m);
        acc += (v + C::BM - 1) / C::BM * p.n_blocks;
      }
      s_prefix[p.num_groups] = acc;
    }
    __syncthreads();
    num_tiles = s_prefix[p.num_groups];
  }

  // XCD-aware rank: workgroups are dealt round-robin over the 8 XCDs, so
  // renumber them to give each XCD a contiguous range of tiles per round.
  const int grid = gridDim.x;
  int rank = blockIdx.x;
  if ((grid & 7) == 0) rank = (blockIdx.x & 7) * (grid >> 3) + (blockIdx.x >> 3);

  int t = rank;
  TileRef cur = next_active<C, KIND>(p, t, grid, num_tiles, s_prefix);
  if (!cur.active) return;
  const LaneOffsets lo = lane_offsets<C>(p.k, wave, lane);
  // Prologue: the first K block of the first tile into stage 0.
  float sb_next = issue_stage<C, 0>(cur, 0, p, wave, wn0, lo);
  int phase = 0;

  WaveTile<C> wt;
  while (cur.active) {
    int t_next = t + grid;
    const TileRef nxt = next_active<C, KIND>(p, t_next, grid, num_tiles, s_prefix);

    bool any_row = false;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) {
      const int r = cur.m0 + wm0 + mt * 16 + (lane & 15);
      bool ok;
      if constexpr (KIND == KIND_CONTIGUOUS) ok = (r < p.m) && (p.aux[r] == cur.group);
      else ok = r < cur.valid_rows;
      wt.row_ok[mt] = ok;
      any_row |= ok;
    }
    wt.on = (__builtin_amdgcn_ballot_w64(any_row) != 0) && (cur.n0 + wn0 < p.n);
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) wt.acc[mt][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    if constexpr (C::STAGES == 2) {
      if (phase == 0) mainloop<C, KIND, 0>(p, cur, nxt, wt, sb_next, wave, wm0, wn0, lane, lo);
      else mainloop<C, KIND, 1>(p, cur, nxt, wt, sb_next, wave, wm0, wn0, lane, lo);
    }
    phase = (phase + k_blocks) % C::STAGES;

    // Epilogue (the next tile's first K block is already in flight): BF16
    // round-to-nearest-even, 8-byte stores of the valid rows.
    if (wt.on) {
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
        if (!wt.row_ok[mt]) continue;
        const int r = cur.m0 + wm0 + mt * 16 + (lane & 15);
        uint16_t* drow = cur.d + (size_t)r * p.n + cur.n0 + wn0 + 4 * (lane >> 4);
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) {
          const f32x4 v = wt.acc[mt][nt];
          uint2 packed;
          packed.x = pack_bf16x2(v[0], v[1]);
          packed.y = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(drow + nt * 16) = packed;
        }
      }
    }
    cur = nxt;
    t = t_next;
  }
  // The last refill loaded a block nobody reads; no wave may end while such
  // a load can still write its LDS.
  wait_vmcnt_0();
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

using CfgLarge = Config<256, 256, 2, 4, 2>;

template <class C, int KIND>
static hipError_t launch(const GemmArgs& args, int num_cus, hipStream_t stream) {
  auto kern = fp8_gemm_nt_kernel<C, KIND>;
  int per_cu = 1;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, C::THREADS, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  const long long slots = (long long)num_cus * per_cu;
  const long long tiles = args.num_tiles;
  int grid = (int)(tiles < slots ? tiles : slots);
  if (grid < 1) return hipSuccess;
  // Keep a large grid a multiple of 8 so that the XCD renumbering applies.
  if (grid > 8) grid -= grid & 7;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::THREADS), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_gemm(int kind, GemmArgs args, int num_cus, hipStream_t stream) {
  using C = CfgLarge;
  args.m_blocks = (args.m + C::BM - 1) / C::BM;
  args.n_blocks = (args.n + C::BN - 1) / C::BN;
  if (kind == KIND_MASKED) {
    // Upper bound for the grid size; the kernel counts the real tiles.
    args.num_tiles = args.num_groups * args.m_blocks * args.n_blocks;
    return launch<C, KIND_MASKED>(args, num_cus, stream);
  }
  if (kind == KIND_CONTIGUOUS) {
    args.num_tiles = C::SLOTS * args.m_blocks * args.n_blocks;
    return launch<C, KIND_CONTIGUOUS>(args, num_cus, stream);
  }
  args.num_tiles = args.m_blocks * args.n_blocks;
  return launch<C, KIND_DENSE>(args, num_cus, stream);
}

}  // namespace dg
