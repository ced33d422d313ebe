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
  int row_limit;       // rows >= row_limit are not addressable (loads clamp)
  int valid_rows;      // dense / masked: rows < valid_rows are written
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
  static constexpr int A_DMA = BM * ROW_BYTES / 1024 / NW;  // 1 KB per wave-wide 16-byte load
  static constexpr int B_DMA = BN * ROW_BYTES / 1024 / NW;
  static constexpr int SA_DMA = WM / 64;                    // 256 B (64 scales) per wave-wide 4-byte load
  static constexpr int LOADS_PER_STAGE = A_DMA + B_DMA + SA_DMA;
  static constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
  static constexpr int SA_BYTES = NW * WM * 4;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SA_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static_assert(BM % (WAVES_M * 16) == 0 && BN % (WAVES_N * 16) == 0, "wave tile");
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns lie in one 128-column scale block");
  static_assert(BM * ROW_BYTES % (1024 * NW) == 0 && BN * ROW_BYTES % (1024 * NW) == 0, "DMA split");
  static_assert(WM % 64 == 0, "scale DMA granularity");
};

// Loads of K block `kb` of one tile into stage S: the A and B tile rows with
// the swizzle of lds_offset(), and each wave's own copy of its rows' scales.
template <class C, int S>
__device__ __forceinline__ void issue_stage(const TileRef& tr, int kb, size_t K, int ld_sfa, int wave, int wm0,
                                            int lane) {
  uint8_t* st = stage_buf<C, S>();
  const size_t kofs = (size_t)kb * BK;
#pragma unroll
  for (int j = 0; j < C::A_DMA; ++j) {
    const int blk = j * C::NW + wave;  // which 1 KB (8 rows) of the A tile
    const int slot = blk * 64 + lane;
    const int row = slot >> 3;
    const int c = (slot & 7) ^ ((row >> 1) & 7);
    const int grow = min(tr.m0 + row, tr.row_limit - 1);
    dma16(tr.a + (size_t)grow * K + kofs + c * 16, st + blk * 1024);
  }
#pragma unroll
  for (int j = 0; j < C::B_DMA; ++j) {
    const int blk = j * C::NW + wave;
    const int slot = blk * 64 + lane;
    const int row = slot >> 3;
    const int c = (slot & 7) ^ ((row >> 1) & 7);
    dma16(tr.b + (size_t)(tr.n0 + row) * K + kofs + c * 16, st + C::A_BYTES + blk * 1024);
  }
#pragma unroll
  for (int j = 0; j < C::SA_DMA; ++j) {
    const int r = min(tr.m0 + wm0 + j * 64 + lane, tr.row_limit - 1);
    dma4(tr.sfa + (size_t)kb * ld_sfa + r, st + C::A_BYTES + C::B_BYTES + (wave * C::WM + j * 64) * 4);
  }
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

template <class C, int KIND>
__global__ void __launch_bounds__(C::THREADS, 1) fp8_gemm_nt_kernel(GemmArgs p) {
  static_assert(C::STAGES >= 2 && C::STAGES <= 4, "pipeline depth");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar scale loads
  const int wave_m = wave / C::WAVES_N;
  const int wave_n = wave % C::WAVES_N;
  const int wm0 = wave_m * C::WM;
  const int wn0 = wave_n * C::WN;
  const int k_blocks = p.k / BK;
  const size_t K = (size_t)p.k;

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

  for (int t = rank; t < num_tiles; t += grid) {
    TileRef tr;
    if constexpr (KIND == KIND_MASKED) {
      int lo = 0, hi = p.num_groups - 1;  // last g with prefix[g] <= t
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
      tr.row_limit = p.m;
      tr.valid_rows = v;
    } else {
      int mb, nb;
      raster(t, p.m_blocks, p.n_blocks, 8, mb, nb);
      tr.m0 = mb * C::BM;
      tr.n0 = nb * C::BN;
      tr.row_limit = p.m;
      tr.valid_rows = p.m;
      tr.a = p.a;
      tr.sfa = p.sfa;
      tr.d = p.d;
      tr.group = 0;
      if constexpr (KIND == KIND_CONTIGUOUS) {
        const int g = p.aux[tr.m0];
        if (g < 0 || g >= p.num_groups) continue;  // a padding block: nothing to compute or write
        tr.group = g;
        tr.b = p.b + (size_t)g * p.n * K;
        tr.sfb = p.sfb + (size_t)g * (p.n / BK) * k_blocks;
      } else {
        tr.b = p.b;
        tr.sfb = p.sfb;
      }
    }

    // Which of this lane's rows are written, and which 16-row bands of this
    // wave hold any written row (bands without one skip their MFMAs).
    bool row_ok[C::MT];
    bool any_row = false;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) {
      const int r = tr.m0 + wm0 + mt * 16 + (lane & 15);
      bool ok;
      if constexpr (KIND == KIND_CONTIGUOUS) ok = (r < p.m) && (p.aux[r] == tr.group);
      else ok = r < tr.valid_rows;
      row_ok[mt] = ok;
      any_row |= ok;
    }
    // A wave whose rows are all invalid skips its MFMAs (it still takes part
    // in the loads and barriers).
    const bool wave_on = __builtin_amdgcn_ballot_w64(any_row) != 0;

    f32x4 acc[C::MT][C::NT];
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) acc[mt][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // The previous tile's stores and stage reads are complete before the
    // stages are refilled.
    wait_vmcnt_0();
    wait_lgkmcnt_0();
    barrier();
    static_for<0, C::STAGES - 1>([&](auto si) {
      constexpr int s = decltype(si)::value;
      if (s < k_blocks) issue_stage<C, s>(tr, s, K, p.ld_sfa, wave, wm0, lane);
    });

    const const_f32_ptr sfb_row = uniform_const_ptr(tr.sfb + (size_t)((tr.n0 + wn0) / BK) * k_blocks);

    for (int kb0 = 0; kb0 < k_blocks; kb0 += C::STAGES) {
      static_for<0, C::STAGES>([&](auto si) {
        constexpr int s = decltype(si)::value;
        const int kb = kb0 + s;
        if (kb >= k_blocks) return;
        wait_stage<C>(C::STAGES - 2);
        wait_lgkmcnt_0();
        barrier();
        // Refill the stage every wave finished reading in the previous step.
        // Near the end of K the last block is loaded again instead of
        // branching around the loads: the stage is not read, and a branch
        // here would make the compiler wait for these loads before reading
        // the current stage.
        issue_stage<C, (s + C::STAGES - 1) % C::STAGES>(tr, min(kb + C::STAGES - 1, k_blocks - 1), K, p.ld_sfa, wave,
                                                        wm0, lane);

        const uint8_t* As = stage_buf<C, s>();
        const uint8_t* Bs = As + C::A_BYTES;
        const float* SAs = reinterpret_cast<const float*>(As + C::A_BYTES + C::B_BYTES) + wave * C::WM;
        const float sb = sfb_row[kb];

        if (!wave_on) return;
        i32x8 bf[C::NT];
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) bf[nt] = read_frag(Bs, wn0 + nt * 16 + (lane & 15), lane);

#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) {
          const i32x8 af = read_frag(As, wm0 + mt * 16 + (lane & 15), lane);
          const float w = SAs[mt * 16 + (lane & 15)] * sb;
          f32x4 part[C::NT];
#pragma unroll
          for (int nt = 0; nt < C::NT; ++nt)
            part[nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[nt], af, (f32x4){0.f, 0.f, 0.f, 0.f}, 0,
                                                                       0, 0, 0, 0, 0);
#pragma unroll
          for (int nt = 0; nt < C::NT; ++nt) acc[mt][nt] += part[nt] * w;
        }
      });
    }

    // Epilogue: BF16 round-to-nearest-even, 8-byte stores of valid rows.
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) {
      if (!row_ok[mt]) continue;
      const int r = tr.m0 + wm0 + mt * 16 + (lane & 15);
      uint16_t* drow = tr.d + (size_t)r * p.n + tr.n0 + wn0 + 4 * (lane >> 4);
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) {
        const f32x4 v = acc[mt][nt];
        uint2 packed;
        packed.x = pack_bf16x2(v[0], v[1]);
        packed.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(drow + nt * 16) = packed;
      }
    }
  }
  // The last K steps re-load a block into a stage nobody reads; no wave may
  // end while such a load can still write its LDS.
  wait_vmcnt_0();
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

using CfgBase = Config<128, 128, 2, 2, 2>;

template <class C, int KIND>
static hipError_t launch(const GemmArgs& args, int num_cus, hipStream_t stream) {
  const size_t lds = 0;  // all LDS is static
  auto kern = fp8_gemm_nt_kernel<C, KIND>;
  int per_cu = 1;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, C::THREADS, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  long long slots = (long long)num_cus * per_cu;
  long long tiles = args.num_tiles;
  int grid = (int)(tiles < slots ? tiles : slots);
  if (grid < 1) return hipSuccess;
  // Keep the grid a multiple of 8 when it is large so the XCD renumbering applies.
  if (grid > 8) grid -= grid & 7;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::THREADS), lds, stream, args);
  return hipGetLastError();
}

hipError_t launch_gemm(int kind, GemmArgs args, int num_cus, hipStream_t stream) {
  using C = CfgBase;
  args.m_blocks = (kind == KIND_MASKED) ? (args.m + C::BM - 1) / C::BM : (args.m + C::BM - 1) / C::BM;
  args.n_blocks = args.n / C::BN;
  if (kind == KIND_MASKED) {
    args.num_tiles = args.num_groups * args.m_blocks * args.n_blocks;  // upper bound; the kernel recounts
    return launch<C, KIND_MASKED>(args, num_cus, stream);
  }
  args.num_tiles = args.m_blocks * args.n_blocks;
  if (kind == KIND_CONTIGUOUS) return launch<C, KIND_CONTIGUOUS>(args, num_cus, stream);
  return launch<C, KIND_DENSE>(args, num_cus, stream);
}

}  // namespace dg
