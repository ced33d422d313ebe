// M-grouped FP8 x FP4 (W4A8) NT GEMM for gfx950 (MI355X): OCP E4M3 A times
// packed OCP E2M1 B, BF16 out ("DeepGEMM Compatibility Wrapper" page, "0.2.7
// Compatibility Additions": the m_grouped_fp8_fp4 entry points with FP8 E4M3
// A, packed E2M1 B, LHS scales per 1x128 and RHS scales per 1x32):
//
//   D[m][n] = bf16( sum_k e4m3(A[m][k]) sa[k/128][m] * e2m1(B[n][k]) sb[k/32][n] )
//
// with power-of-two scales: each float32 scale stands for 2^(e - 127), e its
// exponent field (the UE8M0 reading of the other *_ue8m0 entry points).
// v_mfma_scale_f32_16x16x128_f8f6f4 multiplies E4M3 by E2M1 directly and
// applies one E8M0 scale per lane and operand: in the FP4 operand lane group
// g = lane / 16 holds K positions 32g .. 32g + 31 of its row (16 bytes, even
// k in the low nibble), so its scale is that row's scale of 32-K block g; the
// FP8 operand takes the row's 128-K scale. The products accumulate in the
// MFMA's float32 accumulator: no separate promotion step.
//
// Layouts: contiguous (per-row group index, 128-row aligned segments) and
// masked (per-group valid-row counts read on the device), with the tile
// scheduler of the FP8 kernels. Per 256 x 256 tile a double-buffered K loop
// loads A (128-byte rows), B (64-byte packed rows), the 256 LHS scales and
// the 4 x 256 RHS scales of the K block straight into LDS.

#include "dg_device.h"

namespace dg {
namespace w4a8 {

struct Cfg {
  static constexpr int BM = 256, BN = 256, SLOTS = BM / 128;
  static constexpr int WAVES_N = 4, NW = 8, THREADS = NW * 64;
  static constexpr int WM = 128, WN = 64, MT = WM / 16, NT = WN / 16;
};
constexpr int B_ROW = BK / 2;                      // packed E2M1 bytes per row and K block
constexpr int A_BYTES = Cfg::BM * ROW_BYTES;       // 32 KB
constexpr int B_BYTES = Cfg::BN * B_ROW;           // 16 KB
constexpr int SA_OFF = A_BYTES + B_BYTES;          // 256 LHS scales
constexpr int SB_OFF = SA_OFF + Cfg::BM * 4;       // 4 x 256 RHS scales: [32-K block][column]
constexpr int STAGE_BYTES = SB_OFF + 4 * Cfg::BN * 4;
static_assert(Cfg::NW == 8 && Cfg::BM == 256 && Cfg::BN == 256, "load split below");

__device__ __forceinline__ uint8_t* lds() {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[2 * STAGE_BYTES];
  return buf;
}
__device__ __forceinline__ uint32_t lds_addr() { return (uint32_t)(uintptr_t)(lds_void*)lds(); }

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_dest(lds_base), 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_dest(lds_base), 4, voff, 0, 0, 0);
}

// Byte offset of 16-byte chunk c (0..3) of packed B row `row` in LDS: rows
// are 64 bytes, chunks XOR-swizzled with (row / 4) % 4 so that the 16 rows a
// fragment read touches per chunk fall on 16 different 16-byte bank slots.
__device__ __forceinline__ int b_offset(int row, int c) { return row * B_ROW + ((c ^ ((row >> 2) & 3)) << 4); }

// Where a tile's operands start (the group's B and RHS scales are located
// from the group index: E2M1 rows are K / 2 bytes, and the RHS scales are
// per 32-K block).
struct Src {
  const uint8_t* a;
  const uint8_t* b;
  const float* sa;
  const float* sb;
  uint32_t a_rows, b_rows;
};

__device__ __forceinline__ Src tile_src(const GemmArgs& p, const TileRef& tr) {
  Src s;
  const size_t K = (size_t)p.k;
  s.a_rows = (uint32_t)min(max(tr.load_rows - tr.m0, 0), Cfg::BM);
  s.b_rows = (uint32_t)min(p.n - tr.n0, Cfg::BN);
  s.a = tr.a + (size_t)tr.m0 * K;
  s.sa = tr.sfa + tr.m0;
  s.b = p.b + ((size_t)tr.group * p.n + tr.n0) * (K / 2);
  s.sb = p.sfb + (size_t)tr.group * (K / 32) * p.ld_sfb + tr.n0;
  return s;
}

// Loads of K block kb into the stage at LDS byte address st. Wave w: A rows
// w * 8 + lane / 8 + 64 j (j < 4, 16 bytes each); B rows 16 i + lane / 4 of
// loads i = 2w, 2w + 1 (16 bytes each); waves 0-3 64 LHS scales each; RHS
// scales: loads i = 2w, 2w + 1 cover 32-K block i / 4, columns 64 (i % 4) ..
// + 63. Rows and columns past the matrix read as zero.
__device__ __forceinline__ void issue_block(const GemmArgs& p, const Src& s, int kb, uint32_t st, int wave,
                                            int lane, uint32_t a_lane_off) {
  const uint32_t K = (uint32_t)p.k;
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(s.a + (size_t)kb * BK, s.a_rows * K);
#pragma unroll
  for (int j = 0; j < 4; ++j) dma16(ra, a_lane_off + (uint32_t)j * 64u * K, st + (j * Cfg::NW + wave) * 1024);
  const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(s.b + (size_t)kb * B_ROW, s.b_rows * (K / 2));
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = 2 * wave + h;
    const int row = 16 * i + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    dma16(rb, (uint32_t)row * (K / 2) + (uint32_t)c * 16u, st + A_BYTES + i * 1024);
  }
  if (wave < 4) {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(s.sa + (size_t)kb * p.ld_sfa, s.a_rows * 4u);
    dma4(rs, (uint32_t)(wave * 64 + lane) * 4u, st + SA_OFF + wave * 256);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = 2 * wave + h;
    const int blk = i >> 2, q = i & 3;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(s.sb + (size_t)(kb * 4 + blk) * p.ld_sfb, s.b_rows * 4u);
    dma4(rs, (uint32_t)(64 * q + lane) * 4u, st + SB_OFF + (blk * Cfg::BN + 64 * q) * 4);
  }
}

// One K block of a wave's 128 x 64 sub-tile from the stage at `st`, bands
// 0 .. NB-1 (the rows of the others are not stored). The A fragment and
// scale of band mt + 1 are read before band mt's MFMAs are issued, so that
// the LDS latency hides behind them.
template <int NB>
__device__ __forceinline__ void block(f32x4 (&acc)[Cfg::MT][Cfg::NT], const uint8_t* st, int wm0, int wn0, int lane) {
  const int r = lane & 15, q = lane >> 4;
  i32x8 bf[Cfg::NT];
  int eb[Cfg::NT];
#pragma unroll
  for (int nt = 0; nt < Cfg::NT; ++nt) {
    const int row = wn0 + nt * 16 + r;
    const i32x4 x = *reinterpret_cast<const i32x4*>(st + A_BYTES + b_offset(row, q));
    bf[nt] = (i32x8){x[0], x[1], x[2], x[3], 0, 0, 0, 0};  // an E2M1 operand uses the first four registers
    eb[nt] = e8m0_code(*reinterpret_cast<const float*>(st + SB_OFF + (q * Cfg::BN + row) * 4));
  }
  auto read_a = [&](int mt, i32x8& af, float& sa) {
    const int row = wm0 + mt * 16 + r;
    const i32x4 x = *reinterpret_cast<const i32x4*>(st + lds_offset(row, q));
    const i32x4 y = *reinterpret_cast<const i32x4*>(st + lds_offset(row, q + 4));
    af = (i32x8){x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    sa = *reinterpret_cast<const float*>(st + SA_OFF + row * 4);
  };
  i32x8 af[2];
  float sa[2];
  read_a(0, af[0], sa[0]);
#pragma unroll
  for (int mt = 0; mt < NB; ++mt) {
    if (mt + 1 < NB) read_a(mt + 1, af[(mt + 1) & 1], sa[(mt + 1) & 1]);
    const int ea = e8m0_code(sa[mt & 1]);
#pragma unroll
    for (int nt = 0; nt < Cfg::NT; ++nt)
      // first operand E2M1 (cbsz 4), second E4M3 (blgp 0)
      acc[mt][nt] =
          __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[nt], af[mt & 1], acc[mt][nt], 4, 0, 0, eb[nt], 0, ea);
    if (mt + 1 < NB) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // the next band's reads first
    __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);                         // this band's scale code
    __builtin_amdgcn_sched_group_barrier(0x008, Cfg::NT, 0);                   // then its MFMAs
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The epilogue's staging area: 16 rows of 128 bytes per wave.
__device__ __forceinline__ uint8_t* epilogue_buf() {
  __shared__ __attribute__((aligned(256))) uint8_t buf[Cfg::NW * 16 * ROW_BYTES];
  return buf;
}

// Writes a wave's finished 128 x 64 sub-tile as BF16 (round to nearest
// even), valid rows only. Each 16-row band goes through the wave's own LDS
// staging area so that every store covers a whole 128-byte row segment (8
// lanes per row): the band is written in the MFMA layout (lane l holds row
// l % 16 and 4 columns of each 16-column block), then read back as 8 lanes
// per row; 16-byte slots are XOR-swizzled by row. Each staging access is a
// vector load or store at one offset from the staging area's own address.
template <int KIND>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const TileRef& cur, const RowMask& cm,
                                           const f32x4 (&acc)[Cfg::MT][Cfg::NT], int wave, int wm0, int wn0,
                                           int lane) {
  static_assert(Cfg::WN * 2 == ROW_BYTES, "one 128-byte row segment per wave and row");
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  uint8_t* const scr = epilogue_buf();
  const int wbase = wave * 16 * ROW_BYTES;
  const int r = lane & 15, q = lane >> 4;
  auto slot_off = [](int row, int sl) { return row * ROW_BYTES + ((sl ^ (row & 7)) << 4); };
#pragma unroll
  for (int mt = 0; mt < Cfg::MT; ++mt) {
    const uint32_t valid = band_rows<Cfg, KIND>(cur, cm, wm0, mt);
    if (valid == 0) continue;
#pragma unroll
    for (int nt = 0; nt < Cfg::NT; ++nt) {
      const f32x4 v = acc[mt][nt];
      const i32x2 packed = {(int)pack_bf16x2(v[0], v[1]), (int)pack_bf16x2(v[2], v[3])};
      // columns 16 nt + 4 q .. + 3: half (q & 1) of 16-byte slot 2 nt + q / 2
      *reinterpret_cast<i32x2*>(scr + (wbase + slot_off(r, 2 * nt + (q >> 1)) + (q & 1) * 8)) = packed;
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = (lane >> 3) + 8 * half;
      const int sl = lane & 7;
      const i32x4 v = *reinterpret_cast<const i32x4*>(scr + (wbase + slot_off(row, sl)));
      if ((valid >> row) & 1) {
        uint16_t* drow = cur.d + (size_t)(cur.m0 + wm0 + mt * 16 + row) * p.n + cur.n0 + wn0 + 8 * sl;
        __builtin_nontemporal_store(v, (global_i32x4*)drow);
      }
    }
  }
}

// The K loop of one tile (bands 0 .. NB-1 of the wave computed). Block i
// has landed for every wave after the wait and barrier at the top of step i
// (each waits for all its loads and stores, then all meet), and nobody reads
// the other stage any more. The wait is explicit: the compiler does not see
// the direct-to-LDS loads (bare LDS addresses), and its barrier waits only
// for what it sees. The last step loads the next tile's first block.
template <int NB>
__device__ __forceinline__ void k_loop(const GemmArgs& p, f32x4 (&acc)[Cfg::MT][Cfg::NT], const Src& src,
                                       const Src& nsrc, bool has_next, bool on, int stage, uint32_t base,
                                       const uint8_t* buf, int wave, int lane, uint32_t a_lane_off, int wm0, int wn0) {
  const int k_blocks = p.k / BK;
  for (int i = 0; i < k_blocks; ++i) {
    const int cs = (stage + i) & 1;
    wait_vmcnt_0();
    __syncthreads();
    if (i + 1 < k_blocks) issue_block(p, src, i + 1, base + (cs ^ 1) * STAGE_BYTES, wave, lane, a_lane_off);
    else if (has_next) issue_block(p, nsrc, 0, base + (cs ^ 1) * STAGE_BYTES, wave, lane, a_lane_off);
    if (on) block<NB>(acc, buf + cs * STAGE_BYTES, wm0, wn0, lane);
  }
}

template <int KIND>
__global__ void __launch_bounds__(Cfg::THREADS, 1) fp8_fp4_gemm_kernel(GemmArgs p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave / Cfg::WAVES_N) * Cfg::WM;
  const int wn0 = (wave % Cfg::WAVES_N) * Cfg::WN;
  const int k_blocks = p.k / BK;

  int num_tiles = p.num_tiles;
  [[maybe_unused]] int* s_prefix = nullptr;
  if constexpr (counts_on_device(KIND)) {
    s_prefix = group_table<Cfg, KIND>(p, tid);
    num_tiles = s_prefix[p.num_groups];
  }

  const int row0 = wave * 8 + (lane >> 3);
  const uint32_t a_lane_off =
      (uint32_t)row0 * (uint32_t)p.k + (uint32_t)(((lane & 7) ^ ((row0 >> 1) & 7)) * 16);  // the same for every j

  const int grid = gridDim.x;
  int rank = blockIdx.x;
  if ((grid & 7) == 0) rank = (blockIdx.x & 7) * (grid >> 3) + (blockIdx.x >> 3);

  const uint32_t base = lds_addr();
  const uint8_t* const buf = lds();
  // The first K block of each tile is loaded during the previous tile's last
  // K step, so that its loads overlap that tile's epilogue.
  int t = rank;
  TileRef cur = next_active<Cfg, KIND>(p, t, grid, num_tiles, s_prefix);
  Src src = tile_src(p, cur);
  int stage = 0;  // the stage holding the current tile's first K block
  if (cur.active) issue_block(p, src, 0, base, wave, lane, a_lane_off);
  while (cur.active) {
    int tn = t + grid;
    const TileRef nxt = next_active<Cfg, KIND>(p, tn, grid, num_tiles, s_prefix);
    const Src nsrc = nxt.active ? tile_src(p, nxt) : src;
    RowMask cm{0, 0};
    if constexpr (KIND == KIND_CONTIGUOUS) cm = row_mask(load_row_groups<Cfg>(p, cur, wm0, lane), cur.group);
    bool any_row;
    if constexpr (KIND == KIND_CONTIGUOUS) any_row = (cm.even | cm.odd) != 0;
    else any_row = cur.valid_rows > cur.m0 + wm0;
    const bool on = any_row && cur.n0 + wn0 < p.n;

    f32x4 acc[Cfg::MT][Cfg::NT];
#pragma unroll
    for (int mt = 0; mt < Cfg::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < Cfg::NT; ++nt) acc[mt][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Masked layout: a wave whose valid rows all lie in its first 2, 4 or 6
    // bands runs a copy of the loop without the MFMAs of the others (chosen
    // per tile, outside the loop; a choice per K block inside it made the
    // kernel four times slower). On masked decode, with most tiles partly
    // filled, this made the kernel 16% faster (12% with the 4-band copy alone).
    if constexpr (KIND == KIND_MASKED) {
      const int bands = uniform_int(min(max((cur.valid_rows - cur.m0 - wm0 + 15) / 16, 0), Cfg::MT));
      if (bands <= 2) k_loop<2>(p, acc, src, nsrc, nxt.active, on, stage, base, buf, wave, lane, a_lane_off, wm0, wn0);
      else if (bands <= 4) k_loop<4>(p, acc, src, nsrc, nxt.active, on, stage, base, buf, wave, lane, a_lane_off, wm0, wn0);
      else if (bands <= 6) k_loop<6>(p, acc, src, nsrc, nxt.active, on, stage, base, buf, wave, lane, a_lane_off, wm0, wn0);
      else k_loop<Cfg::MT>(p, acc, src, nsrc, nxt.active, on, stage, base, buf, wave, lane, a_lane_off, wm0, wn0);
    } else {
      for (int i = 0; i < k_blocks; ++i) {
        const int cs = (stage + i) & 1;
        // As in k_loop() (kept inline here: as a call it made this layout 4% slower).
        wait_vmcnt_0();
        __syncthreads();
        if (i + 1 < k_blocks) issue_block(p, src, i + 1, base + (cs ^ 1) * STAGE_BYTES, wave, lane, a_lane_off);
        else if (nxt.active) issue_block(p, nsrc, 0, base + (cs ^ 1) * STAGE_BYTES, wave, lane, a_lane_off);
        if (on) block<Cfg::MT>(acc, buf + cs * STAGE_BYTES, wm0, wn0, lane);
      }
    }
    stage = (stage + k_blocks) & 1;

    if (on) store_tile<KIND>(p, cur, cm, acc, wave, wm0, wn0, lane);
    cur = nxt;
    src = nsrc;
    t = tn;
  }
  wait_vmcnt_0();
}

}  // namespace w4a8

hipError_t launch_fp8_fp4(int kind, GemmArgs args, int num_cus, hipStream_t stream) {
  using namespace w4a8;
  args.m_blocks = (args.m + Cfg::BM - 1) / Cfg::BM;
  args.n_blocks = (args.n + Cfg::BN - 1) / Cfg::BN;
  void (*kern)(GemmArgs);
  if (kind == KIND_MASKED) {
    args.num_tiles = args.num_groups * args.m_blocks * args.n_blocks;  // upper bound; counted on the device
    kern = fp8_fp4_gemm_kernel<KIND_MASKED>;
  } else {
    args.num_tiles = Cfg::SLOTS * args.m_blocks * args.n_blocks;
    kern = fp8_fp4_gemm_kernel<KIND_CONTIGUOUS>;
  }
  int per_cu = 1;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, Cfg::THREADS, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  const int grid = balanced_grid(args.num_tiles, (long long)num_cus * per_cu);
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(Cfg::THREADS), 0, stream, args);
  return hipGetLastError();
}

}  // namespace dg
