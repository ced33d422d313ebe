// FP8 (OCP E4M3) NT GEMM with 1x128 LHS / 128x128 RHS float32 scales and BF16
// output, dense and M-grouped (contiguous, masked), for gfx950 (MI355X): the
// pipeline for long K (see launch_gemm() in dg_kernel.hip for the choice).
//
// The same tiles, scheduler, MFMA, promotion and BF16 epilogue as the
// one-barrier pipeline of dg_kernel.hip ("DeepGEMM for PPU" README,
// "Optimizations": promotion overlapped with data movement and MMA; one
// scheduler for all layouts). What differs is how far ahead the operands
// are loaded: each K block is loaded as two groups (the B tile with the first
// half of the A tile, and the second half of the A tile), and each group's
// LDS is refilled as soon as every wave has read it, behind one of two
// barriers per K step. Every load is thus issued one and a half K steps
// before it is read instead of about one, which hides more of the latency of
// loads that miss the L2 (the long-K grouped workloads stream more operand
// data than the L2 holds); the second barrier costs a little on short K.

#include "dg_device.h"

namespace dg {
namespace deep {

typedef int i32x2 __attribute__((ext_vector_type(2)));

// One wave-wide 16-byte buffer load per lane into LDS from byte offset
// voff + soff (soff wave-uniform, in a scalar register): lane l writes LDS
// byte address lds_base + 16 * l (lds_base is the same for the whole wave).
__device__ __forceinline__ void buf_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_dest(lds_base), 16, voff, (int)soff, 0, 0);
}
// The same with 4 bytes per lane: lane l writes lds_base + 4 * l.
__device__ __forceinline__ void buf_dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_dest(lds_base), 4, voff, (int)soff, 0, 0);
}

// Tile shape and LDS layout. 8 waves as WAVES_M x WAVES_N; wave (wm, wn)
// computes tile rows [wm * WM, +WM) and columns [wn * WN, +WN) in 16-row
// bands of NT 16x16 MFMA blocks.
//
// Each K block's operands are loaded in two groups, so that each group's LDS
// can be refilled as soon as the K loop has read it:
//   group X: the B tile, A half 0 (bands 0-3 of both wave rows: tile rows
//            wm * WM + [0, 64)), their LHS scales, and the RHS scales;
//   group Y: A half 1 (bands 4-7: tile rows wm * WM + [64, 128)) and its
//            LHS scales.
// Every wave issues X_LOADS loads for group X and Y_LOADS for group Y.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct Config {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int THREADS = NW * 64;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int MT = WM / 16, NT = WN / 16;
  static constexpr int SLOTS = BM / 128;  // contiguous layout: 128-row segment blocks per tile row block
  static constexpr int A_DMA = BM * ROW_BYTES / 1024 / NW;  // 1 KB per wave-wide 16-byte load
  static constexpr int B_DMA = BN * ROW_BYTES / 1024 / NW;
  static constexpr int A_HALF_BYTES = BM / 2 * ROW_BYTES;
  static constexpr int B_BYTES = BN * ROW_BYTES;
  static constexpr int SA_HALF_BYTES = BM / 2 * 4;
  // Group X region: B | A half 0 | LHS scales half 0 | RHS scales (64 copies
  // per 128-column block of the tile).
  static constexpr int X_A_OFF = B_BYTES;
  static constexpr int X_SA_OFF = X_A_OFF + A_HALF_BYTES;
  static constexpr int X_SB_OFF = X_SA_OFF + SA_HALF_BYTES;
  static constexpr int X_BYTES = X_SB_OFF + BN / 128 * 256;
  // Group Y region: A half 1 | LHS scales half 1.
  static constexpr int Y_SA_OFF = A_HALF_BYTES;
  static constexpr int Y_BYTES = Y_SA_OFF + SA_HALF_BYTES;
  static constexpr int X_LOADS = B_DMA + A_DMA / 2 + 2;
  static constexpr int Y_LOADS = A_DMA / 2 + 1;
  static_assert(NW == 8 && WAVES_M == 2 && WM == 128 && A_DMA == 4, "A halves: load j covers tile rows [64 j, +64)");
  static_assert(BM % 128 == 0, "tile rows are whole 128-row blocks");
  static_assert(BN % (WAVES_N * 16) == 0, "wave tile");
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns lie in one 128-column scale block");
  static_assert(B_DMA % 2 == 0, "B loads split in halves");
};

// The LDS regions of stage S: R = 0 group X, R = 1 group Y.
template <class C, int S, int R>
__device__ __forceinline__ uint8_t* region() {
  static_assert(S < 2 && R < 2, "stage and region");
  __shared__ __attribute__((aligned(256))) uint8_t buf[R == 0 ? C::X_BYTES : C::Y_BYTES];
  return buf;
}

// LDS byte address of a region (the variable's own address, cast once).
template <class C, int S, int R>
__device__ __forceinline__ uint32_t region_addr() {
  return (uint32_t)(uintptr_t)(lds_void*)region<C, S, R>();
}

// Epilogue staging: ROWS rows of 128 bytes per wave.
template <class C, int ROWS>
__device__ __forceinline__ uint8_t* epilogue_buf() {
  __shared__ __attribute__((aligned(256))) uint8_t buf[C::NW * ROWS * ROW_BYTES];
  return buf;
}

// Per-lane byte offsets of this lane's loads within a tile, fixed for the
// kernel: row * K + 16 * chunk for the A and B tile loads (the j-th load of a
// wave adds j * NW * 8 rows), and 4 * row for the LHS scale load of half 0
// (half 1: 64 rows further).
struct LaneOffsets {
  uint32_t ab;
  uint32_t ab_step;    // bytes between a wave's consecutive tile loads (uniform)
  uint32_t sa, sa_s;   // 4 * lane, and the wave-uniform rest of the scale offset
};

template <class C>
__device__ __forceinline__ LaneOffsets lane_offsets(int k, int wave, int lane) {
  LaneOffsets o;
  const int row0 = wave * 8 + (lane >> 3);
  const int c = (lane & 7) ^ ((row0 >> 1) & 7);  // the same for every load of the wave (NW * 8 % 16 == 0)
  o.ab = (uint32_t)row0 * (uint32_t)k + (uint32_t)c * 16u;
  o.ab_step = (uint32_t)(C::NW * 8) * (uint32_t)k;
  // LHS scales of half h: the 64 rows wm * WM + 64 h + lane of the wave's own
  // wave row wm (the WAVES_N waves of a wave row load the same values).
  o.sa = (uint32_t)lane * 4u;
  o.sa_s = (uint32_t)((wave / C::WAVES_N) * C::WM) * 4u;
  return o;
}

// Global sources of one tile's K blocks, fixed for the tile: A and B at K
// block 0 (the loads of block kb start kb * 128 bytes further), the LHS
// scales at block 0 (kb * ld_sfa floats further), this wave's RHS scale row,
// and the byte extents past which loads read as zero.
struct TileSrc {
  const uint8_t* a;
  const uint8_t* b;
  const float* sa;
  const float* sb;
  uint32_t a_bytes, b_bytes, sa_bytes;
};

template <class C>
__device__ __forceinline__ TileSrc tile_src(const TileRef& tr, const GemmArgs& p, int wn0) {
  TileSrc r;
  const uint32_t K = (uint32_t)p.k;
  const uint32_t a_rows = (uint32_t)min(max(tr.load_rows - tr.m0, 0), C::BM);
  const uint32_t b_rows = (uint32_t)min(p.n - tr.n0, C::BN);
  r.a = uniform_ptr(tr.a + (size_t)tr.m0 * K);
  r.b = uniform_ptr(tr.b + (size_t)tr.n0 * K);
  r.sa = uniform_ptr(tr.sfa + tr.m0);
  r.sb = uniform_ptr(tr.sfb + (size_t)((min(tr.n0 + wn0, p.n - 1)) / BK) * (p.k / BK));
  r.a_bytes = uniform_int(a_rows * K);
  r.b_bytes = uniform_int(b_rows * K);
  r.sa_bytes = uniform_int(a_rows * 4u);
  return r;
}

// Buffer descriptors of K block `kb` of one tile.
struct StageSrc {
  __amdgpu_buffer_rsrc_t a, b, sa, sb;
  uint32_t sb_off;
};

__device__ __forceinline__ StageSrc stage_src(const TileSrc& t, int kb, int ld_sfa, int k_blocks) {
  StageSrc r;
  r.a = buffer_rsrc(t.a + (size_t)kb * BK, t.a_bytes);
  r.b = buffer_rsrc(t.b + (size_t)kb * BK, t.b_bytes);
  r.sa = buffer_rsrc(t.sa + (size_t)kb * ld_sfa, t.sa_bytes);
  r.sb = buffer_rsrc(t.sb, (uint32_t)k_blocks * 4u);
  r.sb_off = (uint32_t)kb * 4u;
  return r;
}

// Group X of one K block into stage S, in three parts: 0 and 1 the B tile
// (rows past the tile's valid columns read as zero), 2 A half 0 (loads 0
// and 2 of the wave: tile rows [0, 64) and [128, 192)), its LHS scales and
// the RHS scale of this wave's columns (one float per wave).
template <class C, int S, int PART>
__device__ __forceinline__ void issue_x(const StageSrc& r, int wave, const LaneOffsets& lo) {
  const uint32_t x = region_addr<C, S, 0>();
  if constexpr (PART < 2) {
#pragma unroll
    for (int j = PART * C::B_DMA / 2; j < (PART + 1) * C::B_DMA / 2; ++j)
      buf_dma16(r.b, lo.ab, j * lo.ab_step, x + (j * C::NW + wave) * 1024);
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      buf_dma16(r.a, lo.ab, (2 * h) * lo.ab_step, x + C::X_A_OFF + (h * C::NW + wave) * 1024);
    buf_dma4(r.sa, lo.sa, lo.sa_s, x + C::X_SA_OFF + (wave / C::WAVES_N) * 256);
    buf_dma4(r.sb, 0u, r.sb_off, x + C::X_SB_OFF + (wave % C::WAVES_N) * C::WN / 128 * 256);
  }
}

// Group Y of one K block into stage S, in two parts: A half 1 (loads 1 and
// 3 of the wave: tile rows [64, 128) and [192, 256)), then its LHS scales.
template <class C, int S, int PART>
__device__ __forceinline__ void issue_y(const StageSrc& r, int wave, const LaneOffsets& lo) {
  const uint32_t y = region_addr<C, S, 1>();
  buf_dma16(r.a, lo.ab, (2 * PART + 1) * lo.ab_step, y + (PART * C::NW + wave) * 1024);
  if constexpr (PART == 1) buf_dma4(r.sa, lo.sa, lo.sa_s + 64u * 4u, y + C::Y_SA_OFF + (wave / C::WAVES_N) * 256);
}

// Buffer descriptors of the K step `ahead` steps after step 0 of the current
// tile: a block of this tile, of the next one, or (with a single K block per
// tile) of the one after. With no such tile the window entries repeat the
// previous one and the loads fetch a block nobody reads.
__device__ __forceinline__ StageSrc refill_src(const TileSrc& t0, const TileSrc& t1, const TileSrc& t2, int ahead,
                                               const GemmArgs& p, int k_blocks) {
  const bool in0 = ahead < k_blocks;
  const bool in1 = ahead < 2 * k_blocks;
  // Field by field (a select between references would put the tiles in memory).
  TileSrc t;
  t.a = in0 ? t0.a : (in1 ? t1.a : t2.a);
  t.b = in0 ? t0.b : (in1 ? t1.b : t2.b);
  t.sa = in0 ? t0.sa : (in1 ? t1.sa : t2.sa);
  t.sb = in0 ? t0.sb : (in1 ? t1.sb : t2.sb);
  t.a_bytes = in0 ? t0.a_bytes : (in1 ? t1.a_bytes : t2.a_bytes);
  t.b_bytes = in0 ? t0.b_bytes : (in1 ? t1.b_bytes : t2.b_bytes);
  t.sa_bytes = in0 ? t0.sa_bytes : (in1 ? t1.sa_bytes : t2.sa_bytes);
  const int kb = in0 ? ahead : (in1 ? ahead - k_blocks : ahead - 2 * k_blocks);
  return stage_src(t, kb, p.ld_sfa, k_blocks);
}

// Per-wave state of the tile being computed.
template <class C>
struct WaveTile {
  f32x4 acc[C::MT][C::NT];
  bool on;  // the wave has a valid row and valid columns: it runs its MFMAs and stores
};

// This lane's LDS byte offsets within a region, fixed for the kernel. Row
// `base + (lane & 15)` of a 16-row band with base a multiple of 16 has swizzle
// ((lane & 15) / 2) % 8, so the two chunks a lane reads sit at the same
// offsets in every band; a band adds 16 rows (2048 bytes), and the region's
// own address is a constant.
struct LdsOffsets {
  uint32_t a0, a1;  // A half: chunk lane/16 and chunk lane/16 + 4 of the wave's first row
  uint32_t b0, b1;  // B: the same for the wave's first column
  uint32_t sa;      // LHS scale half: the wave's first row
};

template <class C>
__device__ __forceinline__ LdsOffsets lds_offsets(int wave_m, int wn0, int lane) {
  LdsOffsets o;
  const int r = lane & 15;
  const uint32_t c0 = (uint32_t)lds_offset(r, lane >> 4);
  const uint32_t c1 = (uint32_t)lds_offset(r, (lane >> 4) + 4);
  o.a0 = (uint32_t)(wave_m * 64) * ROW_BYTES + c0;
  o.a1 = (uint32_t)(wave_m * 64) * ROW_BYTES + c1;
  o.b0 = (uint32_t)wn0 * ROW_BYTES + c0;
  o.b1 = (uint32_t)wn0 * ROW_BYTES + c1;
  o.sa = 4u * (uint32_t)(wave_m * 64 + r);  // + 64 bytes per band
  return o;
}

__device__ __forceinline__ i32x8 frag_pair(const uint8_t* p0, const uint8_t* p1) {
  const i32x4 x = *reinterpret_cast<const i32x4*>(p0);
  const i32x4 y = *reinterpret_cast<const i32x4*>(p1);
  return (i32x8){x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

// The MFMA operand of one lane for one 128-wide K block: 32 bytes of one tile
// row, chunks lane/16 and lane/16 + 4, which the MFMA takes as K positions
// 32*(lane/16) .. +31. Both operands use the same lane -> K mapping, so every
// product still pairs equal k and the block's dot product is unchanged (only
// the order of the MFMA's internal sum moves).
template <class C, int S>
__device__ __forceinline__ i32x8 frag_b(const LdsOffsets& o, int nt) {
  const uint8_t* x = region<C, S, 0>();
  return frag_pair(x + o.b0 + nt * 16 * ROW_BYTES, x + o.b1 + nt * 16 * ROW_BYTES);
}
// Band MT's A fragment: bands 0-3 in group X's A half, 4-7 in group Y's.
template <class C, int S, int MT>
__device__ __forceinline__ i32x8 frag_a(const LdsOffsets& o) {
  const uint8_t* h = MT < 4 ? region<C, S, 0>() + C::X_A_OFF : region<C, S, 1>();
  constexpr int off = (MT % 4) * 16 * ROW_BYTES;
  return frag_pair(h + o.a0 + off, h + o.a1 + off);
}
// LHS scale of band MT's row wm * WM + 16 MT + lane % 16: entry
// 16 (MT % 4) + lane % 16 of wave row wm's 64 entries in its half.
template <class C, int S, int MT>
__device__ __forceinline__ float sa_at(const LdsOffsets& o) {
  const uint8_t* h = MT < 4 ? region<C, S, 0>() + C::X_SA_OFF : region<C, S, 1>() + C::Y_SA_OFF;
  return *reinterpret_cast<const float*>(h + o.sa + (MT % 4) * 16 * 4);
}
template <class C, int S>
__device__ __forceinline__ float sb_at(int wave) {
  return *reinterpret_cast<const float*>(region<C, S, 0>() + C::X_SB_OFF + (wave % C::WAVES_N) * C::WN / 128 * 256);
}

// Rows per pass of the epilogue. The masked and no-padding layouts keep
// their group table in LDS too and stage half bands.
template <int KIND>
constexpr int epilogue_rows() {
  return counts_on_device(KIND) ? 8 : 16;
}

// Writes one finished tile of a wave as BF16 (round to nearest even). Each
// band goes through this wave's own LDS staging area in passes of ER rows, so
// that every store covers a whole 128-byte row segment (8 lanes per row)
// instead of 32-byte pieces: a pass is written in the MFMA layout (lane l
// holds row l % 16 and 4 columns of each 16-column block), then read back as
// 8 lanes per row. 16-byte slots are XOR-swizzled by row.
template <class C, int KIND>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const TileRef& cur, const RowMask& cm,
                                           const WaveTile<C>& wt, int wave, int wm0, int wn0, int lane) {
  static_assert(C::WN * 2 == ROW_BYTES, "one 128-byte row segment per wave and row");
  constexpr int ER = epilogue_rows<KIND>();
  // The lane index is recomputed here, so that the address arithmetic below
  // is not hoisted out of the K loop into registers live across it.
  lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(lane));
  // Each access is one offset from the staging area's own address (a longer
  // chain of pointer arithmetic would hide from the compiler which LDS
  // variable is accessed, and it would then wait for every load into LDS in
  // flight before each access).
  uint8_t* const scr = epilogue_buf<C, ER>();
  const int wbase = wave * ER * ROW_BYTES;
  const int r = lane & 15, g = lane >> 4;
  auto slot_off = [](int row, int sl) { return row * ROW_BYTES + ((sl ^ (row & 7)) << 4); };
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) {
    const uint32_t valid = band_rows<C, KIND>(cur, cm, wm0, mt);
#pragma unroll
    for (int pass = 0; pass < 16 / ER; ++pass) {
      const uint32_t pv = (valid >> (pass * ER)) & ((1u << ER) - 1u);
      if (pv == 0) continue;
      if (ER == 16 || (r / ER) == pass) {
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) {
          const f32x4 v = wt.acc[mt][nt];
          const i32x2 packed = {(int)pack_bf16x2(v[0], v[1]), (int)pack_bf16x2(v[2], v[3])};
          // columns 16 nt + 4 g .. + 3: half (g & 1) of 16-byte slot 2 nt + g / 2
          *reinterpret_cast<i32x2*>(scr + (wbase + slot_off(r % ER, 2 * nt + (g >> 1)) + (g & 1) * 8)) = packed;
        }
      }
#pragma unroll
      for (int half = 0; half < ER / 8; ++half) {
        const int row = (lane >> 3) + 8 * half;
        const int sl = lane & 7;
        const i32x4 q = *reinterpret_cast<const i32x4*>(scr + (wbase + slot_off(row, sl)));
        if ((pv >> row) & 1) {
          uint16_t* drow = cur.d + (size_t)(cur.m0 + wm0 + mt * 16 + pass * ER + row) * p.n + cur.n0 + wn0 + 8 * sl;
          // A global (not flat) store, which the LDS counter does not track, and
          // non-temporal: the output is not read again by this kernel.
          __builtin_nontemporal_store(q, (global_i32x4*)drow);
        }
      }
    }
  }
}

// The MFMA operands of the K step being computed, read from LDS during the
// previous step (or the prologue): B fragments, the ring of A fragments and
// LHS scales (band mt in slot mt % 4, read two bands ahead), and the RHS
// scale.
template <class C>
struct Operands {
  i32x8 bf[C::NT];
  i32x8 af[4];
  float sav[4];
  float sb;
};

template <class C, int S>
__device__ __forceinline__ void read_first(Operands<C>& o, const LdsOffsets& lds, int wave) {
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) o.bf[nt] = frag_b<C, S>(lds, nt);
  o.af[0] = frag_a<C, S, 0>(lds);
  o.sav[0] = sa_at<C, S, 0>(lds);
  o.af[1] = frag_a<C, S, 1>(lds);
  o.sav[1] = sa_at<C, S, 1>(lds);
  o.sb = sb_at<C, S>(wave);
}

// One K step of the global step sequence (over all of this CTA's tiles);
// step g reads stage S = g % 2 and has two barriers:
//   bands 0-1: the A fragment and scale two bands ahead, 4 MFMAs, promotion;
//   band 2:    its MFMAs, then barrier 1: every wave's group Y of step g has
//              landed, and no wave reads group X of stage S any more; group
//              X of step g + 2 is issued into it over bands 2-4;
//   bands 3-5: as bands 0-1;
//   bands 6-7: column by column: the first MFMAs, then barrier 2: every
//              wave's group X of step g + 1 has landed, and no wave reads
//              group Y of stage S any more; group Y of step g + 2 is issued
//              into it; B fragment nt of step g + 1 is read as soon as its
//              last MFMA of step g has issued, then the next step's first A
//              fragments and scales.
// Each load is thus issued one and a half K steps before the barrier after
// which it is read. At each barrier the loads of exactly one K step (X_LOADS
// + Y_LOADS per wave) may still be in flight: vector memory loads complete
// in order, so waiting for that count covers every older load (stores and
// other loads in between only make the wait stricter). The MFMAs issued
// before each barrier keep the matrix core busy while the waves meet.
constexpr int BAND_A = 2;  // band of barrier 1

// The MFMAs of band mt. Float32 scales: the partial sums of the K block go
// to `part`, promoted by the caller. Power-of-two scales (E8): the MFMA
// applies them as E8M0 block scales (eb for the B fragments, this band's ea
// for the A fragment) and accumulates into the totals itself.
template <class C, bool E8, int MT>
__device__ __forceinline__ void band_mfmas(WaveTile<C>& wt, f32x4 (&part)[C::NT], const Operands<C>& o, int eb) {
  if constexpr (E8) {
    const int ea = e8m0_code(o.sav[MT % 4]);
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt)
      wt.acc[MT][nt] = mfma_fp8_scaled(o.bf[nt], o.af[MT % 4], wt.acc[MT][nt], eb, ea);
  } else {
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt)
      part[nt] = mfma_fp8(o.bf[nt], o.af[MT % 4], (f32x4){0.f, 0.f, 0.f, 0.f});
  }
}

template <class C, int S, bool E8>
__device__ __forceinline__ void step_on(WaveTile<C>& wt, Operands<C>& o, const StageSrc& r2, int wave,
                                        const LdsOffsets& lds, const LaneOffsets& lo) {
  static_assert(C::MT == 8 && C::NT == 4, "pipeline shape");
  constexpr int SN = 1 - S;
  constexpr int IN_FLIGHT = C::X_LOADS + C::Y_LOADS;
  const float sb = o.sb;
  [[maybe_unused]] const int eb = e8m0_code(sb);
  static_for<0, 6>([&](auto mi) {
    constexpr int mt = decltype(mi)::value;
    f32x4 part[C::NT];
    if constexpr (mt == BAND_A) {
      band_mfmas<C, E8, mt>(wt, part, o, eb);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<IN_FLIGHT>();
      wait_lgkmcnt_0();
      barrier();
      __builtin_amdgcn_sched_barrier(0);
      o.af[(mt + 2) % 4] = frag_a<C, S, mt + 2>(lds);
      o.sav[(mt + 2) % 4] = sa_at<C, S, mt + 2>(lds);
      issue_x<C, S, 0>(r2, wave, lo);
      if constexpr (!E8) {
        const float w = o.sav[mt % 4] * sb;
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) wt.acc[mt][nt] += part[nt] * w;
      }
      __builtin_amdgcn_sched_barrier(0);
    } else {
      o.af[(mt + 2) % 4] = frag_a<C, S, mt + 2>(lds);
      o.sav[(mt + 2) % 4] = sa_at<C, S, mt + 2>(lds);
      if constexpr (mt == BAND_A + 1) issue_x<C, S, 1>(r2, wave, lo);
      if constexpr (mt == BAND_A + 2) issue_x<C, S, 2>(r2, wave, lo);
      band_mfmas<C, E8, mt>(wt, part, o, eb);
      if constexpr (!E8) {
        const float w = o.sav[mt % 4] * sb;
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) wt.acc[mt][nt] += part[nt] * w;
      }
      // Issue order: the reads two bands ahead and this band's share of the
      // refill first, then the MFMAs, then the promotion.
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // DS reads
      if constexpr (mt == BAND_A + 1) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // VMEM loads
      if constexpr (mt == BAND_A + 2) __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);
      if constexpr (E8) __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // VALU: the scale code
      __builtin_amdgcn_sched_group_barrier(0x008, C::NT, 0);  // MFMA
      if constexpr (!E8) __builtin_amdgcn_sched_group_barrier(0x002, 4 * C::NT + 1, 0);  // VALU
      __builtin_amdgcn_sched_barrier(0);
    }
  });
  const float w6 = o.sav[6 % 4] * sb;
  const float w7 = o.sav[7 % 4] * sb;
  [[maybe_unused]] const int ea6 = e8m0_code(o.sav[6 % 4]);
  [[maybe_unused]] const int ea7 = e8m0_code(o.sav[7 % 4]);
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) {
    f32x4 p6, p7;
    if constexpr (E8) {
      wt.acc[6][nt] = mfma_fp8_scaled(o.bf[nt], o.af[6 % 4], wt.acc[6][nt], eb, ea6);
      wt.acc[7][nt] = mfma_fp8_scaled(o.bf[nt], o.af[7 % 4], wt.acc[7][nt], eb, ea7);
    } else {
      p6 = mfma_fp8(o.bf[nt], o.af[6 % 4], (f32x4){0.f, 0.f, 0.f, 0.f});
      p7 = mfma_fp8(o.bf[nt], o.af[7 % 4], (f32x4){0.f, 0.f, 0.f, 0.f});
    }
    __builtin_amdgcn_sched_barrier(0);
    if (nt == 0) {
      wait_vmcnt<IN_FLIGHT>();
      wait_lgkmcnt_0();
      barrier();
      __builtin_amdgcn_sched_barrier(0);
      issue_y<C, S, 0>(r2, wave, lo);
    }
    if (nt == 1) issue_y<C, S, 1>(r2, wave, lo);
    // The next step's operands (at a tile's last step: the next tile's first).
    o.bf[nt] = frag_b<C, SN>(lds, nt);
    if (nt == 0) o.sb = sb_at<C, SN>(wave);
    if (nt == 1) {
      o.af[0] = frag_a<C, SN, 0>(lds);
      o.sav[0] = sa_at<C, SN, 0>(lds);
    }
    if (nt == 3) {
      o.af[1] = frag_a<C, SN, 1>(lds);
      o.sav[1] = sa_at<C, SN, 1>(lds);
    }
    if constexpr (!E8) {
      wt.acc[6][nt] += p6 * w6;
      wt.acc[7][nt] += p7 * w7;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// A step of a wave with nothing to compute in the current tile: its share of
// the loads and the barriers, then the next step's operands.
template <class C, int S>
__device__ __forceinline__ void step_off(Operands<C>& o, const StageSrc& r2, int wave,
                                         const LdsOffsets& lds, const LaneOffsets& lo) {
  constexpr int IN_FLIGHT = C::X_LOADS + C::Y_LOADS;
  wait_vmcnt<IN_FLIGHT>();
  wait_lgkmcnt_0();
  barrier();
  issue_x<C, S, 0>(r2, wave, lo);
  issue_x<C, S, 1>(r2, wave, lo);
  issue_x<C, S, 2>(r2, wave, lo);
  wait_vmcnt<IN_FLIGHT>();
  wait_lgkmcnt_0();
  barrier();
  issue_y<C, S, 0>(r2, wave, lo);
  issue_y<C, S, 1>(r2, wave, lo);
  read_first<C, 1 - S>(o, lds, wave);
}

template <class C, int KIND>
__device__ __forceinline__ bool tile_on(const GemmArgs& p, const TileRef& cur, const RowMask& cm, int wm0, int wn0) {
  bool any_row;
  if constexpr (KIND == KIND_CONTIGUOUS) any_row = (cm.even | cm.odd) != 0;
  else any_row = cur.valid_rows > cur.m0 + wm0;
  return any_row && (cur.n0 + wn0 < p.n);
}

template <class C>
__device__ __forceinline__ void zero_acc(WaveTile<C>& wt) {
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) wt.acc[mt][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
}

// The K loop of one tile; its first step reads stage PHASE (the global step
// sequence runs on across tiles, so a tile with an odd number of K blocks
// leaves the next one starting on the other stage).
template <class C, int KIND, int PHASE, bool E8>
__device__ __forceinline__ void tile_loop(const GemmArgs& p, const TileSrc& t0, const TileSrc& t1, const TileSrc& t2,
                                          WaveTile<C>& wt, int wave, const LdsOffsets& lds,
                                          const LaneOffsets& lo) {
  const int k_blocks = p.k / BK;
  Operands<C> op;
  read_first<C, PHASE>(op, lds, wave);
  for (int kb0 = 0; kb0 < k_blocks; kb0 += 2) {
    static_for<0, 2>([&](auto si) {
      constexpr int S = (decltype(si)::value + PHASE) % 2;
      const int kb = kb0 + decltype(si)::value;
      if (kb >= k_blocks) return;
      // The refills are issued unconditionally (past the last tile they load
      // a block nobody reads).
      const StageSrc r2 = refill_src(t0, t1, t2, kb + 2, p, k_blocks);
      if (wt.on) step_on<C, S, E8>(wt, op, r2, wave, lds, lo);
      else step_off<C, S>(op, r2, wave, lds, lo);
    });
  }
}

template <class C, int KIND, bool E8>
__global__ void __launch_bounds__(C::THREADS, 1) fp8_gemm_nt_kernel(GemmArgs p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar scale loads
  const int wave_m = wave / C::WAVES_N;
  const int wave_n = wave % C::WAVES_N;
  const int wm0 = wave_m * C::WM;
  const int wn0 = wave_n * C::WN;
  const int k_blocks = p.k / BK;

  // The masked and no-padding layouts count their tiles on the device.
  int num_tiles = p.num_tiles;
  [[maybe_unused]] int* s_prefix = nullptr;
  if constexpr (counts_on_device(KIND)) {
    s_prefix = group_table<C, KIND>(p, tid);
    num_tiles = s_prefix[p.num_groups];
  }

  // XCD-aware rank: workgroups are dealt round-robin over the 8 XCDs, so
  // renumber them to give each XCD a contiguous range of tiles per round.
  const int grid = gridDim.x;
  int rank = blockIdx.x;
  if ((grid & 7) == 0) rank = (blockIdx.x & 7) * (grid >> 3) + (blockIdx.x >> 3);

  // A window of three tiles: the current one and the next two (refills run
  // two K steps ahead, which reaches the tile after next when a tile has a
  // single K block). Missing tiles repeat the previous window entry.
  int t = rank;
  TileRef cur = next_active<C, KIND>(p, t, grid, num_tiles, s_prefix);
  if (!cur.active) return;
  int t1 = t + grid;
  TileRef nxt = next_active<C, KIND>(p, t1, grid, num_tiles, s_prefix);
  int t2 = t1 + grid;
  TileRef nx2;
  nx2.active = false;
  if (nxt.active) nx2 = next_active<C, KIND>(p, t2, grid, num_tiles, s_prefix);
  const LaneOffsets lo = lane_offsets<C>(p.k, wave, lane);
  const LdsOffsets lds = lds_offsets<C>(wave_m, wn0, lane);
  TileSrc c0 = tile_src<C>(cur, p, wn0);
  TileSrc c1 = nxt.active ? tile_src<C>(nxt, p, wn0) : c0;
  TileSrc c2 = nx2.active ? tile_src<C>(nx2, p, wn0) : c1;

  // The first tile's row groups (contiguous layout) are loaded before the
  // prologue's loads, so that waiting for them never waits for those.
  [[maybe_unused]] RowGroups rg{-1, -1};
  if constexpr (KIND == KIND_CONTIGUOUS) rg = load_row_groups<C>(p, cur, wm0, lane);

  // Prologue: the loads in the order of the steady state up to barrier 2 of
  // step -1 (groups X and Y of step 0, group X of step 1), that barrier (its
  // wait: group X of step 0 has landed), then group Y of step 1.
  {
    const StageSrc r0 = refill_src(c0, c1, c2, 0, p, k_blocks);
    const StageSrc r1 = refill_src(c0, c1, c2, 1, p, k_blocks);
    issue_x<C, 0, 0>(r0, wave, lo);
    issue_x<C, 0, 1>(r0, wave, lo);
    issue_x<C, 0, 2>(r0, wave, lo);
    issue_y<C, 0, 0>(r0, wave, lo);
    issue_y<C, 0, 1>(r0, wave, lo);
    issue_x<C, 1, 0>(r1, wave, lo);
    issue_x<C, 1, 1>(r1, wave, lo);
    issue_x<C, 1, 2>(r1, wave, lo);
    wait_vmcnt<C::X_LOADS + C::Y_LOADS>();
    barrier();
    issue_y<C, 1, 0>(r1, wave, lo);
    issue_y<C, 1, 1>(r1, wave, lo);
  }
  int phase = 0;

  RowMask cmask{0, 0};
  if constexpr (KIND == KIND_CONTIGUOUS) cmask = row_mask(rg, cur.group);

  WaveTile<C> wt;
  while (cur.active) {
    wt.on = tile_on<C, KIND>(p, cur, cmask, wm0, wn0);
    if constexpr (KIND == KIND_CONTIGUOUS) rg = load_row_groups<C>(p, nxt, wm0, lane);
    zero_acc(wt);
    if (phase == 0) tile_loop<C, KIND, 0, E8>(p, c0, c1, c2, wt, wave, lds, lo);
    else tile_loop<C, KIND, 1, E8>(p, c0, c1, c2, wt, wave, lds, lo);
    phase = (phase + k_blocks) % 2;

    // The next tile's row mask: its row groups were loaded when this tile
    // started, before at least a K step of refills.
    [[maybe_unused]] RowMask nmask{0, 0};
    if constexpr (KIND == KIND_CONTIGUOUS) {
      int e = rg.even, o = rg.odd;
      asm volatile("" : "+v"(e), "+v"(o));  // keeps the compare (and its wait) here
      nmask = row_mask(RowGroups{e, o}, nxt.group);
    }
    // Epilogue: the next tile's loads are in flight into the stages; the
    // output goes through the separate staging area.
    if (wt.on) store_tile<C, KIND>(p, cur, cmask, wt, wave, wm0, wn0, lane);
    // Slide the window.
    cmask = nmask;
    cur = nxt;
    c0 = c1;
    nxt = nx2;
    c1 = c2;
    if (nx2.active) {
      t2 += grid;
      nx2 = next_active<C, KIND>(p, t2, grid, num_tiles, s_prefix);
    }
    c2 = nx2.active ? tile_src<C>(nx2, p, wn0) : c1;
  }
  // The last refills loaded blocks nobody reads; no wave may end while such
  // a load can still write its LDS.
  wait_vmcnt_0();
}

// ---------------------------------------------------------------------------
// Launcher
// ---------------------------------------------------------------------------

using CfgLarge = Config<256, 256, 2, 4>;

template <class C, int KIND>
static hipError_t launch(const GemmArgs& args, int num_cus, hipStream_t stream) {
  auto kern = args.scale_e8m0 ? fp8_gemm_nt_kernel<C, KIND, true> : fp8_gemm_nt_kernel<C, KIND, false>;
  int per_cu = 1;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, C::THREADS, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  const int grid = balanced_grid(args.num_tiles, (long long)num_cus * per_cu);
  if (grid < 1) return hipSuccess;
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
  if (kind == KIND_NOPAD) {
    // Upper bound: each group adds at most one partial row block.
    args.num_tiles = (args.m_blocks + args.num_groups) * args.n_blocks;
    return launch<C, KIND_NOPAD>(args, num_cus, stream);
  }
  if (kind == KIND_CONTIGUOUS) {
    args.num_tiles = C::SLOTS * args.m_blocks * args.n_blocks;
    return launch<C, KIND_CONTIGUOUS>(args, num_cus, stream);
  }
  args.num_tiles = args.m_blocks * args.n_blocks;
  return launch<C, KIND_DENSE>(args, num_cus, stream);
}

}  // namespace deep
}  // namespace dg
