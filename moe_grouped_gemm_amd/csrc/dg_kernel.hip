// FP8 (OCP E4M3) NT GEMM with 1x128 LHS / 128x128 RHS float32 scales and BF16
// output, dense and M-grouped (contiguous, masked), for gfx950 (MI355X).
//
// One persistent kernel serves the three layouts ("DeepGEMM for PPU" README,
// "Optimizations": one block scheduler for the non-grouped and grouped
// kernels, rasterised for L2 reuse). Per output tile and per 128-wide K block:
//
//   1. HBM -> LDS: the A tile [BM][128] and B tile [BN][128] bytes and the
//      tile's LHS scales, with 16-byte direct-to-LDS buffer loads, into one
//      of two stages (the loads of a block are issued one to two K steps
//      before it is read);
//   2. matrix cores: one v_mfma_f32_16x16x128_f8f6f4 per 16x16 sub-tile gives
//      the block's float32 partial sum;
//   3. promotion: total += partial * (sfa[m] * sfb[n/128]) in float32
//      ("Persistent warp-specialization": promotion overlapped with data
//      movement and MMA);
//   4. after the last K block, BF16 round-to-nearest-even and store of the
//      rows that are valid for the layout (staged through LDS into whole
//      128-byte row segments).
//
// The MFMA is issued with the B fragment as its first operand and the A
// fragment as its second, so that each lane's four results share one output
// row m (lane % 16) and four consecutive columns: one LHS scale per lane per
// 16-row band.

#include "dg_device.h"

namespace dg {

// One LDS buffer per pipeline stage.
template <class C, int S>
__device__ __forceinline__ uint8_t* stage_buf() {
  static_assert(S < C::STAGES, "stage index");
  __shared__ __attribute__((aligned(1024))) uint8_t buf[C::STAGE_BYTES];
  return buf;
}

// LDS byte address of stage S (the variable's own address, cast once).
template <class C, int S>
__device__ __forceinline__ uint32_t stage_addr() {
  return (uint32_t)(uintptr_t)(lds_void*)stage_buf<C, S>();
}

// One wave-wide 16-byte buffer load per lane into LDS: lane l writes LDS byte
// address lds_base + 16 * l (lds_base is the same for the whole wave).
__device__ __forceinline__ void buf_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_dest(lds_base), 16, voff, 0, 0, 0);
}
// The same with 4 bytes per lane: lane l writes lds_base + 4 * l.
__device__ __forceinline__ void buf_dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_dest(lds_base), 4, voff, 0, 0, 0);
}

// Per-lane byte offsets of this lane's loads within a tile, fixed for the
// kernel: row * K + 16 * chunk for the A and B tile loads (the j-th load of a
// wave adds j * NW * 8 rows), and 4 * row for the scale load.
struct LaneOffsets {
  uint32_t ab;
  uint32_t ab_step;    // bytes between a wave's consecutive tile loads
  uint32_t sa;
};

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

// The loads of one K block into stage S are issued in four parts (see the K
// loop for when): part 0 and 1 the A tile (rows past the tile's valid rows
// read as zero), part 2 and 3 the B tile (both with the swizzle of
// lds_offset()), part 3 also the tile's LHS scales and the RHS scale of this
// wave's columns (returned; usable once the stage has been waited for).

template <class C, int S, int PART>
__device__ __forceinline__ float issue_part(const StageSrc& r, int wave, const LaneOffsets& lo) {
  static_assert(C::A_DMA % 2 == 0 && C::B_DMA % 2 == 0, "loads split in halves");
  const uint32_t st = stage_addr<C, S>();
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

// Position of tile row r's LHS scale in a stage's scale area.
template <class C>
__device__ __forceinline__ int sa_index(int r) {
  return (r / C::SA_ROWS) * 64 + r % C::SA_ROWS;
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
  bool on;    // the wave has a valid row and valid columns: it runs its MFMAs and stores
  int bands;  // masked and no-padding layouts: 16-row bands up to the wave's last valid row
};

// A wave whose valid rows lie in its first HALF_BANDS bands runs a copy of
// the K loop without the other bands' MFMAs (their rows are never stored).
// In a masked decode batch most 256-row tiles are partly filled; on such a
// workload this cut the kernel time by 10% (float32 scales).
constexpr int HALF_BANDS = 4;

// This lane's LDS byte offsets within a stage, fixed for the kernel. Row
// `base + (lane & 15)` of a 16-row band with base a multiple of 16 has swizzle
// ((lane & 15) / 2) % 8, so the two chunks a lane reads sit at the same
// offsets in every band; a band adds 16 rows (2048 bytes), and the stage
// buffer's own address is a constant.
struct LdsOffsets {
  uint32_t a0, a1;  // A rows: chunk lane/16 and chunk lane/16 + 4 of the wave's band 0
  uint32_t b0, b1;  // B rows: the same for the wave's first 16 columns
  uint32_t sa;      // the LHS scale of the wave's band 0 row
};

template <class C>
__device__ __forceinline__ LdsOffsets lds_offsets(int wm0, int wn0, int lane) {
  LdsOffsets o;
  const int r = lane & 15;
  const uint32_t c0 = (uint32_t)lds_offset(r, lane >> 4);
  const uint32_t c1 = (uint32_t)lds_offset(r, (lane >> 4) + 4);
  o.a0 = (uint32_t)wm0 * ROW_BYTES + c0;
  o.a1 = (uint32_t)wm0 * ROW_BYTES + c1;
  o.b0 = (uint32_t)C::A_BYTES + (uint32_t)wn0 * ROW_BYTES + c0;
  o.b1 = (uint32_t)C::A_BYTES + (uint32_t)wn0 * ROW_BYTES + c1;
  o.sa = (uint32_t)(C::A_BYTES + C::B_BYTES) + 4u * (uint32_t)sa_index<C>(wm0 + r);
  return o;
}

// The MFMA operand of one lane for one 128-wide K block: 32 bytes of one tile
// row, chunks lane/16 and lane/16 + 4, which the MFMA takes as K positions
// 32*(lane/16) .. +31. Both operands use the same lane -> K mapping, so every
// product still pairs equal k and the block's dot product is unchanged (only
// the order of the MFMA's internal sum moves).
template <class C, int S>
__device__ __forceinline__ i32x8 frag_at(uint32_t off0, uint32_t off1, int band) {
  const uint8_t* st = stage_buf<C, S>();
  const i32x4 x = *reinterpret_cast<const i32x4*>(st + off0 + band * 16 * ROW_BYTES);
  const i32x4 y = *reinterpret_cast<const i32x4*>(st + off1 + band * 16 * ROW_BYTES);
  return (i32x8){x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

// LHS scale of band `mt`'s row: rows wm0 + 16 mt + r, with wm0 a multiple of
// SA_ROWS = 32, sit (mt / 2) regions and (mt % 2) * 16 entries after band 0's.
template <class C, int S>
__device__ __forceinline__ float sa_at(uint32_t off, int mt) {
  static_assert(C::SA_ROWS == 32, "scale layout");
  const uint8_t* st = stage_buf<C, S>();
  return *reinterpret_cast<const float*>(st + off + 4 * ((mt / 2) * 64 + (mt % 2) * 16));
}

// Writes one finished tile of a wave as BF16 (round to nearest even). Each
// 16-row band goes through LDS so that every store covers whole 128-byte row
// segments (8 lanes per row) instead of 32-byte pieces: the band is written
// in the MFMA layout (lane l holds row l % 16 and 4 columns of each
// 16-column block) into two of this wave's own 1 KB B-tile slots of stage S,
// the stage the tile's last step read; no wave reads that stage again before
// the next barrier, and only this wave's own refill loads, issued later,
// overwrite these slots. 16-byte slots are XOR-swizzled by row.
//
// Each staging access is a vector load or store at one offset from the stage
// buffer's own address: the compiler then knows which LDS variable it
// touches (a struct-typed or longer pointer chain loses that, and it would
// wait for every load in flight before each access).
template <class C, int KIND, int S>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const TileRef& cur, const RowMask& cm,
                                           const WaveTile<C>& wt, int wave, int wm0, int wn0, int lane) {
  static_assert(C::WN * 2 == 128 && C::B_DMA >= 2, "one 128-byte row segment per wave and band");
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  uint8_t* const st = stage_buf<C, S>();
  const int wbase = C::A_BYTES + wave * 1024;  // slot j of the wave at + j * NW * 1024
  const int r = lane & 15, g = lane >> 4;
  auto slot_off = [](int row, int sl) { return (row >> 3) * C::NW * 1024 + (row & 7) * 128 + ((sl ^ (row & 7)) << 4); };
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) {
    const uint32_t valid = band_rows<C, KIND>(cur, cm, wm0, mt);
    if (valid == 0) continue;
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      const f32x4 v = wt.acc[mt][nt];
      const i32x2 packed = {(int)pack_bf16x2(v[0], v[1]), (int)pack_bf16x2(v[2], v[3])};
      // columns 16 nt + 4 g .. + 3: half (g & 1) of 16-byte slot 2 nt + g / 2
      *reinterpret_cast<i32x2*>(st + (wbase + slot_off(r, 2 * nt + (g >> 1)) + (g & 1) * 8)) = packed;
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = (lane >> 3) + 8 * half;
      const int sl = lane & 7;
      const i32x4 q = *reinterpret_cast<const i32x4*>(st + (wbase + slot_off(row, sl)));
      if ((valid >> row) & 1) {
        uint16_t* drow = cur.d + (size_t)(cur.m0 + wm0 + mt * 16 + row) * p.n + cur.n0 + wn0 + 8 * sl;
        // A global (not flat) store, which the LDS counter does not track.
        // Non-temporal for the grouped layouts (plain stores made masked decode
        // 10% slower); plain for the dense GEMM, 2-3% faster there.
        if constexpr (KIND == KIND_DENSE) *(global_i32x4*)drow = q;
        else __builtin_nontemporal_store(q, (global_i32x4*)drow);
      }
    }
  }
}

// The K loop of one tile; its first step reads stage PHASE. Step g of the
// global sequence of K steps reads stage s = g % 2:
//   entry:     the first step's operands are read (its stage was completed
//              before the last barrier);
//   bands 0-5: the A fragment and scale two bands ahead from stage s, 4
//              MFMAs, the promotion of the band; bands 0 and 1 also issue
//              parts 2 and 3 of the refill of stage 1 - s (step g + 1);
//   barrier:   after it every wave's loads of step g + 1 have landed and no
//              wave reads stage s any more (bands 6 and 7 work from
//              registers);
//   bands 6-7: column by column, so that B fragment nt is re-read for step
//              g + 1 as soon as its last MFMA of step g has issued, then
//              the next step's first A fragments; parts 0 and 1 of the
//              refill of stage s (step g + 2) are issued.
// The MFMAs issued before the barrier keep the matrix core busy while the
// waves meet, and every step starts with its operands in registers. Only
// bands below NB are computed (NB < 8: neither their A fragments are read
// nor their MFMAs issued); the loads and barriers are the same for every NB.
template <class C, int KIND, int PHASE, bool E8, int NB>
__device__ __forceinline__ void mainloop(const GemmArgs& p, const TileSrc& t0, const TileSrc& t1, const TileSrc& t2,
                                         WaveTile<C>& wt, float (&sbv)[2], int wave, const LdsOffsets& lds,
                                         const LaneOffsets& lo, const RowGroups& nrg, int ngroup, RowMask& nmask) {
  static_assert(C::STAGES == 2 && C::MT == 8 && C::NT == 4, "pipeline shape");
  static_assert(NB == C::MT || (NB >= 2 && NB <= 6), "a partial copy computes bands 0 .. NB-1 before the barrier");
  // The next tile's row mask (contiguous layout), after a barrier: see RowGroups.
  auto next_rows = [&]() {
    if constexpr (KIND == KIND_CONTIGUOUS) {
      int e = nrg.even, o = nrg.odd;
      asm volatile("" : "+v"(e), "+v"(o));  // keeps the compare (and the wait for the loads) here
      nmask = row_mask(RowGroups{e, o}, ngroup);
    }
  };
  const int k_blocks = p.k / BK;
  i32x8 af[4];    // A ring: band mt's fragment in slot mt % 4
  float sav[4];   // LHS scale ring, same slots
  i32x8 bf[C::NT];
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) bf[nt] = frag_at<C, PHASE>(lds.b0, lds.b1, nt);
  af[0] = frag_at<C, PHASE>(lds.a0, lds.a1, 0);
  sav[0] = sa_at<C, PHASE>(lds.sa, 0);
  af[1] = frag_at<C, PHASE>(lds.a0, lds.a1, 1);
  sav[1] = sa_at<C, PHASE>(lds.sa, 1);
  for (int kb0 = 0; kb0 < k_blocks; kb0 += C::STAGES) {
    static_for<0, C::STAGES>([&](auto si) {
      constexpr int step = decltype(si)::value;
      constexpr int s = (step + PHASE) % C::STAGES;
      constexpr int sn = (s + 1) % C::STAGES;
      const int kb = kb0 + step;
      if (kb >= k_blocks) return;
      // The refills are issued unconditionally (past the last tile they load
      // a block nobody reads): a branch here would make the compiler wait
      // for them before reading the current stage.
      const StageSrc r1 = refill_src(t0, t1, t2, kb + 1, p, k_blocks);
      const StageSrc r2 = refill_src(t0, t1, t2, kb + 2, p, k_blocks);
      const float sb = sbv[s];  // this step's RHS scale, loaded with its stage
      [[maybe_unused]] const int eb = e8m0_code(sb);
      if (!wt.on) {
        issue_part<C, sn, 2>(r1, wave, lo);
        sbv[sn] = issue_part<C, sn, 3>(r1, wave, lo);
        wait_vmcnt_0();
        wait_lgkmcnt_0();
        barrier();
        next_rows();
        issue_part<C, s, 0>(r2, wave, lo);
        issue_part<C, s, 1>(r2, wave, lo);
        return;
      }

#pragma unroll
      for (int mt = 0; mt < 6; ++mt) {
        if (mt + 2 < NB) {
          af[(mt + 2) % 4] = frag_at<C, s>(lds.a0, lds.a1, mt + 2);
          sav[(mt + 2) % 4] = sa_at<C, s>(lds.sa, mt + 2);
        }
        if (mt == 0) issue_part<C, sn, 2>(r1, wave, lo);
        if (mt == 1) sbv[sn] = issue_part<C, sn, 3>(r1, wave, lo);
        if (mt >= NB) {  // folded at compile time (the loop is unrolled)
          __builtin_amdgcn_sched_barrier(0);
          continue;
        }
        if constexpr (E8) {
          // Power-of-two scales: the MFMA applies them and accumulates.
          const int ea = e8m0_code(sav[mt % 4]);
#pragma unroll
          for (int nt = 0; nt < C::NT; ++nt)
            wt.acc[mt][nt] = mfma_fp8_scaled(bf[nt], af[mt % 4], wt.acc[mt][nt], eb, ea);
        } else {
          f32x4 part[C::NT];
#pragma unroll
          for (int nt = 0; nt < C::NT; ++nt)
            part[nt] = mfma_fp8(bf[nt], af[mt % 4], (f32x4){0.f, 0.f, 0.f, 0.f});
          const float w = sav[mt % 4] * sb;
#pragma unroll
          for (int nt = 0; nt < C::NT; ++nt) wt.acc[mt][nt] += part[nt] * w;
        }
        // Issue order: the reads two bands ahead and this band's share of
        // the refill first, then the MFMAs, then the promotion.
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // DS reads
        if (mt == 0) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // VMEM loads
        if (mt == 1) __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);
        if constexpr (E8) __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // VALU: the scale code
        __builtin_amdgcn_sched_group_barrier(0x008, C::NT, 0);  // MFMA
        if constexpr (!E8) __builtin_amdgcn_sched_group_barrier(0x002, 4 * C::NT + 1, 0);  // VALU
        __builtin_amdgcn_sched_barrier(0);
      }
      const float w6 = sav[6 % 4] * sb;
      const float w7 = sav[7 % 4] * sb;
      [[maybe_unused]] const int ea6 = e8m0_code(sav[6 % 4]);
      [[maybe_unused]] const int ea7 = e8m0_code(sav[7 % 4]);
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) {
        f32x4 p6, p7;
        if constexpr (NB == C::MT) {
          if constexpr (E8) {
            wt.acc[6][nt] = mfma_fp8_scaled(bf[nt], af[6 % 4], wt.acc[6][nt], eb, ea6);
            wt.acc[7][nt] = mfma_fp8_scaled(bf[nt], af[7 % 4], wt.acc[7][nt], eb, ea7);
          } else {
            p6 = mfma_fp8(bf[nt], af[6 % 4], (f32x4){0.f, 0.f, 0.f, 0.f});
            p7 = mfma_fp8(bf[nt], af[7 % 4], (f32x4){0.f, 0.f, 0.f, 0.f});
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (nt == 0) {
          wait_lgkmcnt_0();
          wait_vmcnt_0();
          barrier();
          next_rows();
          __builtin_amdgcn_sched_barrier(0);
          issue_part<C, s, 0>(r2, wave, lo);
        }
        if (nt == 1) issue_part<C, s, 1>(r2, wave, lo);
        // The next step's operands (past a tile's last step: the next
        // tile's first, which its entry reads again).
        bf[nt] = frag_at<C, sn>(lds.b0, lds.b1, nt);
        if (nt == 1) {
          af[0] = frag_at<C, sn>(lds.a0, lds.a1, 0);
          sav[0] = sa_at<C, sn>(lds.sa, 0);
        }
        if (nt == 3) {
          af[1] = frag_at<C, sn>(lds.a0, lds.a1, 1);
          sav[1] = sa_at<C, sn>(lds.sa, 1);
        }
        if constexpr (!E8 && NB == C::MT) {
          wt.acc[6][nt] += p6 * w6;
          wt.acc[7][nt] += p7 * w7;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
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
  const LdsOffsets lds = lds_offsets<C>(wm0, wn0, lane);
  TileSrc c0 = tile_src<C>(cur, p, wn0);
  TileSrc c1 = nxt.active ? tile_src<C>(nxt, p, wn0) : c0;
  TileSrc c2 = nx2.active ? tile_src<C>(nx2, p, wn0) : c1;

  // The first tile's row groups (contiguous layout) are loaded before the
  // prologue's loads, so that waiting for them never waits for those.
  [[maybe_unused]] RowGroups crg{-1, -1};
  if constexpr (KIND == KIND_CONTIGUOUS) crg = load_row_groups<C>(p, cur, wm0, lane);

  // Prologue: step 0 into stage 0 and parts 0 and 1 of step 1 into stage 1
  // (the first step issues the rest); step 0 must have landed for every wave
  // before it is read.
  float sbv[2];
  {
    const StageSrc r0 = refill_src(c0, c1, c2, 0, p, k_blocks);
    const StageSrc r1 = refill_src(c0, c1, c2, 1, p, k_blocks);
    issue_part<C, 0, 0>(r0, wave, lo);
    issue_part<C, 0, 1>(r0, wave, lo);
    issue_part<C, 0, 2>(r0, wave, lo);
    sbv[0] = issue_part<C, 0, 3>(r0, wave, lo);
    issue_part<C, 1, 0>(r1, wave, lo);
    issue_part<C, 1, 1>(r1, wave, lo);
    sbv[1] = 0.f;
    wait_vmcnt<C::A_DMA>();  // all but the last A_DMA loads (step 1's parts 0 and 1)
    barrier();
  }
  int phase = 0;

  RowMask cmask{0, 0}, nmask{0, 0};
  if constexpr (KIND == KIND_CONTIGUOUS) cmask = row_mask(crg, cur.group);

  WaveTile<C> wt;
  while (cur.active) {
    bool any_row;
    if constexpr (KIND == KIND_CONTIGUOUS) any_row = (cmask.even | cmask.odd) != 0;
    else any_row = cur.valid_rows > cur.m0 + wm0;
    wt.on = any_row && (cur.n0 + wn0 < p.n);
    wt.bands = C::MT;
    if constexpr (counts_on_device(KIND))
      wt.bands = uniform_int(min(max((cur.valid_rows - cur.m0 - wm0 + 15) / 16, 0), C::MT));
    RowGroups nrg{-1, -1};
    if constexpr (KIND == KIND_CONTIGUOUS) nrg = load_row_groups<C>(p, nxt, wm0, lane);
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) wt.acc[mt][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    if (counts_on_device(KIND) && wt.bands <= HALF_BANDS) {
      if (phase == 0) mainloop<C, KIND, 0, E8, HALF_BANDS>(p, c0, c1, c2, wt, sbv, wave, lds, lo, nrg, nxt.group, nmask);
      else mainloop<C, KIND, 1, E8, HALF_BANDS>(p, c0, c1, c2, wt, sbv, wave, lds, lo, nrg, nxt.group, nmask);
    } else {
      if (phase == 0) mainloop<C, KIND, 0, E8, C::MT>(p, c0, c1, c2, wt, sbv, wave, lds, lo, nrg, nxt.group, nmask);
      else mainloop<C, KIND, 1, E8, C::MT>(p, c0, c1, c2, wt, sbv, wave, lds, lo, nrg, nxt.group, nmask);
    }
    phase = (phase + k_blocks) % C::STAGES;

    // Epilogue (the next tile's first K block has landed, its second is in
    // flight), from the stage the tile's last step read.
    if (wt.on) {
      if (phase == 0) store_tile<C, KIND, 1>(p, cur, cmask, wt, wave, wm0, wn0, lane);
      else store_tile<C, KIND, 0>(p, cur, cmask, wt, wave, wm0, wn0, lane);
    }
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
// Launchers
// ---------------------------------------------------------------------------

using CfgLarge = Config<256, 256, 2, 4, 2>;

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
  if (args.k / BK >= DEEP_MIN_K_BLOCKS) return deep::launch_gemm(kind, args, num_cus, stream);
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

}  // namespace dg
