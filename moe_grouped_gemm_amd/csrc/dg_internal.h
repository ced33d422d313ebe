// Internal interface between the C ABI (dg_api.cpp) and the kernels
// (dg_kernel.hip). Not installed; not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

enum { KIND_DENSE = 0, KIND_CONTIGUOUS = 1, KIND_MASKED = 2, KIND_NOPAD = 3 };

// Layouts whose tiles the kernel finds from per-group row counts read on the
// device (a group table in LDS, see group_table()).
constexpr bool counts_on_device(int kind) { return kind == KIND_MASKED || kind == KIND_NOPAD; }

// Size of the group table in LDS: the masked layout keeps G + 1 tile
// prefixes, the no-padding layout G + 1 tile prefixes and G + 1 row offsets.
constexpr int GROUP_TABLE_INTS = 4098;
constexpr int MAX_MASKED_GROUPS = GROUP_TABLE_INTS - 2;
constexpr int MAX_NOPAD_GROUPS = GROUP_TABLE_INTS / 2 - 1;

// Kernel arguments, passed by value. Byte pointers: A and B are E4M3 codes,
// D is BF16 bits.
struct GemmArgs {
  const uint8_t* a;
  const float* sfa;
  const uint8_t* b;
  const float* sfb;
  uint16_t* d;
  const int32_t* aux;  // contiguous: grouped_layout[m]; masked: masked_m[G]; no-padding: rows of
                       // each group [G]; dense: unused
  int m;               // dense/contiguous/no-padding: rows of A and D; masked: max_m
  int n, k, num_groups;
  int ld_sfa;          // leading dimension of the transposed LHS scales
  int ld_sfb;          // FP8 x FP4 GEMMs only: leading dimension of the per-32-K RHS scales
  int scale_e8m0;      // nonzero: every scale is used as 2^(its exponent field - 127), applied
                       // by the MFMA itself (E8M0 block scales) instead of a float32 promotion
  int m_blocks, n_blocks, num_tiles;  // filled in by launch_gemm
};

// Enqueues the FP8 x FP4 (W4A8) grouped GEMM of layout `kind` (contiguous or
// masked) on `stream` (dg_kernel_fp4.hip); arguments already validated.
hipError_t launch_fp8_fp4(int kind, GemmArgs args, int num_cus, hipStream_t stream);

// Largest group count of the K-grouped GEMM (its group offsets travel in the
// kernel arguments).
constexpr int MAX_KGROUPED_GROUPS = 512;

// Arguments of the K-grouped GEMM (dg_kernel_kgrouped.hip), passed by value.
struct KGroupedArgs {
  const uint8_t* a;    // [m][k] E4M3
  const float* sfa;    // [k/128][ld_sfa]
  const uint8_t* b;    // [n][k] E4M3
  const float* sfb;    // [k/128][ld_sfb]
  const float* c;      // [G][m][n] or null (then D is the product alone); may equal d
  float* d;            // [G][m][n]
  int m, n, k;         // k: the total K, also the row stride of A and B
  int num_groups;
  int ld_sfa, ld_sfb;
  int scale_e8m0;                          // nonzero: scales read as E8M0 and applied by the MFMA
  int m_blocks, n_blocks, num_tiles;       // filled in by launch_k_grouped
  int k_off[MAX_KGROUPED_GROUPS + 1];      // first K block of each group; k_off[G] = k / 128
};

hipError_t launch_k_grouped(KGroupedArgs& args, int num_cus, hipStream_t stream);

// Persistent grid size for `tiles` tiles on `slots` resident workgroups: the
// fewest workgroups that need no more rounds of tiles than `slots` would,
// above 8 rounded up to a multiple of 8 (so that the kernels' XCD
// renumbering applies) and capped at `slots`. Fewer workgroups with the same number of
// rounds measured faster on MI355X (448 tiles: 224 workgroups beat 256 by
// 3-6%): less contention and power draw, same critical path.
inline int balanced_grid(long long tiles, long long slots) {
  if (tiles <= 0 || slots <= 0) return 0;
  const long long rounds = (tiles + slots - 1) / slots;
  long long g = (tiles + rounds - 1) / rounds;
  if (g > 8) g = (g + 7) / 8 * 8;
  return (int)(g < slots ? g : slots);
}

// Enqueues the kernel for `kind` on `stream`; arguments already validated.
hipError_t launch_gemm(int kind, GemmArgs args, int num_cus, hipStream_t stream);

// K blocks from which launch_gemm() uses the pipeline of dg_kernel_deep.hip,
// which loads operands further ahead (measured on MI355X: 4-4.5% faster on
// the K = 7168 grouped workloads, 2-3% slower at K = 2048).
constexpr int DEEP_MIN_K_BLOCKS = 32;

namespace deep {
hipError_t launch_gemm(int kind, GemmArgs args, int num_cus, hipStream_t stream);
}

}  // namespace dg
