// Internal interface between the C ABI (dg_api.cpp) and the kernels
// (dg_kernel.hip). Not installed; not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

enum { KIND_DENSE = 0, KIND_CONTIGUOUS = 1, KIND_MASKED = 2 };

// Largest group count of the masked layout (the per-group tile prefix lives in LDS).
constexpr int MAX_MASKED_GROUPS = 4096;

// Kernel arguments, passed by value. Byte pointers: A and B are E4M3 codes,
// D is BF16 bits.
struct GemmArgs {
  const uint8_t* a;
  const float* sfa;
  const uint8_t* b;
  const float* sfb;
  uint16_t* d;
  const int32_t* aux;  // contiguous: grouped_layout[m]; masked: masked_m[G]; dense: unused
  int m;               // dense/contiguous: rows of A and D; masked: max_m
  int n, k, num_groups;
  int ld_sfa;          // leading dimension of the transposed LHS scales
  int m_blocks, n_blocks, num_tiles;  // filled in by launch_gemm
};

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
