// K-grouped FP8 (OCP E4M3) NT GEMM for gfx950 (MI355X): the weight-gradient
// shape of an MoE layer ("DeepGEMM Compatibility Wrapper" page, "0.2.7
// Compatibility Additions": contiguous K-grouped FP8 NT GEMM with host-side
// K sizes, each a multiple of 128, scale recipe (1, 1, 128), and a float32
// C that is cleared, copied or accumulated in place).
//
// The K axis is split into consecutive groups; group g owns K blocks
// [k_off[g], k_off[g + 1]) of A [M][K] and B [N][K] (row stride K) and has
// its own float32 output D[g] [M][N]:
//
//   D[g][m][n] = C[g][m][n] + sum over k in group g of
//                e4m3(A[m][k]) sfa[k/128][m] * e4m3(B[n][k]) sfb[k/128][n]
//
// Both operands carry one float32 scale per row and 128-wide K block, stored
// transposed (sfa [K/128][align4(M)], sfb [K/128][align4(N)]).
//
// One persistent kernel walks all groups' 256 x 256 output tiles, group by
// group. Per tile it runs a double-buffered K loop over the group's blocks:
// the direct-to-LDS 16-byte buffer loads of block i + 1 are issued right
// after the barrier that frees their stage, then block i is multiplied (one
// v_mfma_f32_16x16x128_f8f6f4 per 16x16 sub-tile, the B fragment as the
// first operand, so a lane's four results share one row and cover four
// consecutive columns) and promoted, one band behind the MFMAs:
// total += partial * (sfa[m] * sfb[n]), where the RHS scale differs per
// column. The float32 totals, plus C, leave through 16-byte buffer stores
// clipped at the tile's last valid row.

#include "dg_device.h"

namespace dg {
namespace kgrouped {

constexpr int BM = 256, BN = 256, WAVES_N = 4, NW = 8, THREADS = NW * 64;
constexpr int WM = 128, WN = 64, MT = WM / 16, NT = WN / 16;
constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
constexpr int SA_OFF = A_BYTES + B_BYTES;  // the tile rows' LHS scales (float32)
constexpr int SB_OFF = SA_OFF + BM * 4;    // the tile columns' RHS scales (float32)
constexpr int STAGE_BYTES = SB_OFF + BN * 4;
constexpr int AB_LOADS = BM * ROW_BYTES / 1024 / NW;  // wave-wide 16-byte loads per operand and wave
static_assert(AB_LOADS == 4 && BM / NW * 2 == 64, "load split");

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

// One output tile: its group, origin, K blocks and real rows / columns.
struct Tile {
  int g, m0, n0, kb0, nkb;
  int a_rows, b_rows;
};

__device__ __forceinline__ Tile tile_at(const KGroupedArgs& p, int t) {
  Tile tl;
  const int per_group = p.m_blocks * p.n_blocks;
  tl.g = t / per_group;
  int mb, nb;
  raster(t - tl.g * per_group, p.m_blocks, p.n_blocks, 4, mb, nb);  // panels of 4: 1% faster than 8, 3% than 16
  tl.m0 = mb * BM;
  tl.n0 = nb * BN;
  tl.kb0 = p.k_off[tl.g];
  tl.nkb = p.k_off[tl.g + 1] - tl.kb0;
  tl.a_rows = min(BM, p.m - tl.m0);
  tl.b_rows = min(BN, p.n - tl.n0);
  return tl;
}

// Issues the loads of K block kb of a tile into the stage at LDS byte
// address `st`. Wave w loads rows w * 8 + lane / 8 + 64 j (j < 4) of the A
// and the B tile, 16 bytes each and chunk-swizzled as lds_offset() reads
// them (lane_off is row * K + 16 * chunk); waves 0-3 also load 64 of the
// tile's LHS scales each, waves 4-7 64 of its RHS scales. Rows and columns
// past the matrix read as zero.
__device__ __forceinline__ void issue_block(const KGroupedArgs& p, const Tile& tl, int kb, uint32_t st, int wave,
                                            int lane, uint32_t lane_off) {
  const uint32_t lda = (uint32_t)p.k;
  const __amdgpu_buffer_rsrc_t ra =
      buffer_rsrc(p.a + (size_t)tl.m0 * lda + (size_t)kb * BK, (uint32_t)tl.a_rows * lda);
  const __amdgpu_buffer_rsrc_t rb =
      buffer_rsrc(p.b + (size_t)tl.n0 * lda + (size_t)kb * BK, (uint32_t)tl.b_rows * lda);
#pragma unroll
  for (int j = 0; j < AB_LOADS; ++j) {
    dma16(ra, lane_off + (uint32_t)j * 64u * lda, st + (j * NW + wave) * 1024);
    dma16(rb, lane_off + (uint32_t)j * 64u * lda, st + A_BYTES + (j * NW + wave) * 1024);
  }
  if (wave < 4) {
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(p.sfa + (size_t)kb * p.ld_sfa + tl.m0, (uint32_t)tl.a_rows * 4u);
    dma4(rs, (uint32_t)(wave * 64 + lane) * 4u, st + SA_OFF + wave * 256);
  } else {
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(p.sfb + (size_t)kb * p.ld_sfb + tl.n0, (uint32_t)tl.b_rows * 4u);
    dma4(rs, (uint32_t)((wave - 4) * 64 + lane) * 4u, st + SB_OFF + (wave - 4) * 256);
  }
}

// This lane's LDS offsets within a stage: the two 16-byte chunks of its
// fragment row (chunks lane/16 and lane/16 + 4 of row lane % 16 of the
// wave's first band / column block), its row's LHS scale and its four
// columns' RHS scales.
struct Offsets {
  uint32_t a0, a1, b0, b1, sa, sb;
  uint32_t sb_row;  // the RHS scale of the B row this lane holds in the MFMA operand
};

// The promotion of one band, deferred: the MFMA partial sums of its four
// 16x16 blocks and their weights sfa[m] * sfb[n].
struct Pending {
  f32x4 part[NT];
  f32x4 w[NT];
};

__device__ __forceinline__ void clear(Pending& pd) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) pd.part[nt] = pd.w[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
}

// One K block of a wave's 128 x 64 sub-tile from the stage at `st`.
// Float32 scales: partial sums promoted with each column's own RHS scale,
// one band behind: band mt's promotion is issued between band mt + 1's
// MFMAs, so it never waits for the MFMA it depends on. Band 0 promotes the
// previous K block's last band, which `pd` carries with its weights (zero
// at a tile's first block); the block's RHS scales are read only after
// that, which keeps both sets of registers from being live at once.
// Power-of-two scales (E8): the MFMA applies them as E8M0 codes, one per
// lane and operand (the B operand's lane holds row lane % 16 of its 16-row
// block, the A operand's likewise), and accumulates into the totals.
template <bool E8>
__device__ __forceinline__ void block(f32x4 (&acc)[MT][NT], const uint8_t* st, const Offsets& o, Pending& pd) {
  i32x8 bf[NT];
  [[maybe_unused]] f32x4 sb[NT];
  [[maybe_unused]] int eb[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const i32x4 x = *reinterpret_cast<const i32x4*>(st + o.b0 + nt * 16 * ROW_BYTES);
    const i32x4 y = *reinterpret_cast<const i32x4*>(st + o.b1 + nt * 16 * ROW_BYTES);
    bf[nt] = (i32x8){x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    if constexpr (E8) eb[nt] = e8m0_code(*reinterpret_cast<const float*>(st + o.sb_row + nt * 64));
  }
  // The A fragment and scale of band mt + 1 are read before band mt's MFMAs
  // are issued, so that the LDS latency hides behind them.
  auto read_a = [&](int mt, i32x8& af, float& sa) {
    const i32x4 x = *reinterpret_cast<const i32x4*>(st + o.a0 + mt * 16 * ROW_BYTES);
    const i32x4 y = *reinterpret_cast<const i32x4*>(st + o.a1 + mt * 16 * ROW_BYTES);
    af = (i32x8){x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    sa = *reinterpret_cast<const float*>(st + o.sa + mt * 64);
  };
  i32x8 af[2];
  float sa[2];
  [[maybe_unused]] f32x4 prev[NT];  // the MFMA partials of band mt - 1
  [[maybe_unused]] float s_prev = 0.f;
  read_a(0, af[0], sa[0]);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt + 1 < MT) read_a(mt + 1, af[(mt + 1) & 1], sa[(mt + 1) & 1]);
    const i32x8 a_cur = af[mt & 1];
    const float s_cur = sa[mt & 1];
    if constexpr (E8) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[mt][nt] = mfma_fp8_scaled(bf[nt], a_cur, acc[mt][nt], eb[nt], e8m0_code(s_cur));
    } else {
      f32x4 part[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        part[nt] = mfma_fp8(bf[nt], a_cur, (f32x4){0.f, 0.f, 0.f, 0.f});
        if (mt == 0) acc[MT - 1][nt] += pd.part[nt] * pd.w[nt];
        else acc[mt - 1][nt] += prev[nt] * (sb[nt] * s_prev);
      }
      if (mt == 0) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sb[nt] = *reinterpret_cast<const f32x4*>(st + o.sb + nt * 64);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) prev[nt] = part[nt];
      s_prev = s_cur;
      if (mt == MT - 1) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          pd.part[nt] = part[nt];
          pd.w[nt] = sb[nt] * s_cur;
        }
      }
    }
    if (mt + 1 < MT) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // the next band's reads first
    if constexpr (E8) {
      __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);   // the scale code
      __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);  // this band's MFMAs
    } else {
      // Each MFMA, then a quarter of the previous band's promotion (band 0:
      // 4 FMAs; later bands 4 multiplications for the weights and 4 FMAs;
      // the last band also the 16 multiplications of its own weights).
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (mt == 0) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        else if (mt == MT - 1) __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
        else __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      }
      if (mt == 0) __builtin_amdgcn_sched_group_barrier(0x100, NT, 0);  // this block's RHS scales
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The deferred promotion of a tile's last band.
__device__ __forceinline__ void flush(f32x4 (&acc)[MT][NT], Pending& pd) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[MT - 1][nt] += pd.part[nt] * pd.w[nt];
  clear(pd);
}

template <bool HAS_C, bool E8>
__global__ void __launch_bounds__(THREADS, 1) k_grouped_kernel(KGroupedArgs p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave / WAVES_N) * WM;
  const int wn0 = (wave % WAVES_N) * WN;

  const int row0 = wave * 8 + (lane >> 3);
  const uint32_t lane_off =
      (uint32_t)row0 * (uint32_t)p.k + (uint32_t)(((lane & 7) ^ ((row0 >> 1) & 7)) * 16);  // same for every j
  const int r = lane & 15, q = lane >> 4;
  Offsets o;
  o.a0 = (uint32_t)(wm0 * ROW_BYTES + lds_offset(r, q));
  o.a1 = (uint32_t)(wm0 * ROW_BYTES + lds_offset(r, q + 4));
  o.b0 = (uint32_t)(A_BYTES + wn0 * ROW_BYTES + lds_offset(r, q));
  o.b1 = (uint32_t)(A_BYTES + wn0 * ROW_BYTES + lds_offset(r, q + 4));
  o.sa = (uint32_t)(SA_OFF + 4 * (wm0 + r));
  o.sb = (uint32_t)(SB_OFF + 4 * (wn0 + 4 * q));
  o.sb_row = (uint32_t)(SB_OFF + 4 * (wn0 + r));

  // XCD-aware rank, as in the other kernels.
  const int grid = gridDim.x;
  int rank = blockIdx.x;
  if ((grid & 7) == 0) rank = (blockIdx.x & 7) * (grid >> 3) + (blockIdx.x >> 3);

  const uint32_t base = lds_addr();
  const uint8_t* const buf = lds();
  // The first K block of a tile is loaded during the previous tile's last K
  // step when there is one (a tile of an empty group has no K step: the next
  // tile then loads its own first block).
  int t = rank;
  int stage = 0;        // the stage that holds (or will hold) the current tile's first block
  bool loaded = false;  // whether the current tile's first block has been issued
  while (t < p.num_tiles) {
    const Tile tl = tile_at(p, t);
    const int tn = t + grid;
    const bool has_next = tn < p.num_tiles;
    const Tile nx = has_next ? tile_at(p, tn) : tl;
    const bool on = tl.m0 + wm0 < p.m && tl.n0 + wn0 < p.n;
    f32x4 acc[MT][NT];
    Pending pd;
    clear(pd);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    if (tl.nkb > 0 && !loaded) {
      wait_vmcnt_0();
      __syncthreads();  // no wave still reads the stage
      issue_block(p, tl, tl.kb0, base + stage * STAGE_BYTES, wave, lane, lane_off);
    }
    bool next_loaded = false;
    for (int i = 0; i < tl.nkb; ++i) {
      const int cs = (stage + i) & 1;
      // Block i has landed for every wave (each waits for its own loads,
      // then all meet), and nobody reads the other stage any more. The
      // wait is explicit: the compiler does not see the direct-to-LDS loads
      // (bare LDS addresses), and its barrier waits only for what it sees.
      wait_vmcnt_0();
      __syncthreads();
      if (i + 1 < tl.nkb) {
        issue_block(p, tl, tl.kb0 + i + 1, base + (cs ^ 1) * STAGE_BYTES, wave, lane, lane_off);
      } else if (has_next && nx.nkb > 0) {
        issue_block(p, nx, nx.kb0, base + (cs ^ 1) * STAGE_BYTES, wave, lane, lane_off);
        next_loaded = true;
      }
      if (on) block<E8>(acc, buf + cs * STAGE_BYTES, o, pd);
    }
    if constexpr (!E8) flush(acc, pd);
    stage = (stage + tl.nkb) & 1;
    loaded = next_loaded;

    if (on) {
      // Buffer loads and stores relative to the tile's first row, clipped
      // at its last valid row: rows past M read as zero and are not
      // written, so the code has no per-lane branches. Two bands at a time,
      // software-pipelined: the C loads of band pair j + 2 are issued right
      // after the stores of pair j, so that waiting for the loads of pair
      // j + 1 never waits for stores (a wave's memory operations complete in
      // issue order). C and D may be one buffer; each element is read and
      // written by this lane only, so reading ahead of the stores is safe.
      typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
      const size_t tile0 = ((size_t)tl.g * p.m + tl.m0) * (size_t)p.n;
      const uint32_t tile_bytes = (uint32_t)tl.a_rows * (uint32_t)p.n * 4u;
      const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(p.d + tile0, tile_bytes);
      [[maybe_unused]] const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(HAS_C ? p.c + tile0 : p.d + tile0, tile_bytes);
      const uint32_t lane_off = ((uint32_t)(wm0 + r) * (uint32_t)p.n + (uint32_t)(tl.n0 + wn0 + 4 * q)) * 4u;
      const uint32_t band_bytes = 16u * (uint32_t)p.n * 4u;
      f32x4 cv[2][2][NT];
      auto load_pair = [&](int j, f32x4 (&c2)[2][NT]) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            if constexpr (HAS_C)
              c2[h][nt] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rc, lane_off + nt * 64, (2 * j + h) * band_bytes, 0));
            else c2[h][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
          }
      };
      load_pair(0, cv[0]);
      load_pair(1, cv[1]);
#pragma unroll
      for (int j = 0; j < MT / 2; ++j) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[2 * j + h][nt] + cv[j & 1][h][nt]),
                                                   rd, lane_off + nt * 64, (2 * j + h) * band_bytes, 0);
        if (j + 2 < MT / 2) load_pair(j + 2, cv[j & 1]);
      }
    }
    t = tn;
  }
  // Loads issued past the last block read: none (every issued block is read).
  wait_vmcnt_0();
}

}  // namespace kgrouped

hipError_t launch_k_grouped(KGroupedArgs& args, int num_cus, hipStream_t stream) {
  using namespace kgrouped;
  args.m_blocks = (args.m + BM - 1) / BM;
  args.n_blocks = (args.n + BN - 1) / BN;
  args.num_tiles = args.num_groups * args.m_blocks * args.n_blocks;
  auto kern = args.scale_e8m0 ? (args.c ? k_grouped_kernel<true, true> : k_grouped_kernel<false, true>)
                              : (args.c ? k_grouped_kernel<true, false> : k_grouped_kernel<false, false>);
  int per_cu = 1;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, THREADS, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  const int grid = balanced_grid(args.num_tiles, (long long)num_cus * per_cu);
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(THREADS), 0, stream, args);
  return hipGetLastError();
}

}  // namespace dg
