// Matrix-core throughput ceiling of the device: the FP8 MFMA loop alone,
// with the launch shape of the GEMM kernels (one workgroup of 8 waves per
// CU, two waves per SIMD) and the same instruction, so that a GEMM's time
// can be compared with what the matrix cores reach on this part at the
// clock they actually run at. Declared in include/dg_ceiling.h.

#include "../../include/dg_ceiling.h"

#include <hip/hip_runtime.h>

#include "dg_device.h"

namespace dg {
namespace {

constexpr int kChains = 16;   // independent accumulators per wave
constexpr int kThreads = 512;

// Each wave keeps kChains 16x16 float32 accumulators and issues
// v_mfma_f32_16x16x128_f8f6f4 on its register fragments iters * kChains
// times (constant-zero scale codes select the unscaled instruction, see
// mfma_fp8 in dg_device.h). PROMOTE 1 adds, per MFMA, the four float32 FMAs
// of the per-128-K promotion of the float32-scale GEMMs (total += part * w),
// one MFMA behind, as the GEMM kernels issue them; PROMOTE 2 that of the
// K-grouped GEMM, whose weights differ per column: four multiplications
// (w = sfb[n] * sfa[m]) and four FMAs per MFMA.
template <int PROMOTE>
__global__ void __launch_bounds__(kThreads, 1) mfma_ceiling_kernel(const i32x4* frag, float* sink, int iters) {
  const int lane = threadIdx.x & 63;
  const i32x4 x0 = frag[lane], x1 = frag[64 + lane], y0 = frag[128 + lane], y1 = frag[192 + lane];
  const i32x8 a = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  const i32x8 b = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
  const float w = __builtin_bit_cast(float, 0x3f800000 | (lane & 7));
  [[maybe_unused]] const f32x4 sb = {w, 0.5f * w, 0.25f * w, 2.f * w};
  [[maybe_unused]] float sa = w;
  f32x4 acc[kChains], tot[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = tot[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
  i32x8 av = a, bv = b;
  for (int it = 0; it < iters; ++it) {
    // The operands count as new values every iteration (as fragments read
    // from LDS would be): nothing computed from them can leave the loop.
    asm volatile("" : "+v"(av), "+v"(bv));
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      if constexpr (PROMOTE > 0) {
        asm volatile("" : "+v"(av));  // a distinct operand per MFMA (no common subexpressions)
        const f32x4 part = mfma_fp8(bv, av, (f32x4){0.f, 0.f, 0.f, 0.f});
        if constexpr (PROMOTE == 1) {
          tot[c] += acc[c] * w;  // the previous MFMA's partial
        } else {
          asm volatile("" : "+v"(sa));  // a new row scale per MFMA: the weights are recomputed
          tot[c] += acc[c] * (sb * sa);
        }
        acc[c] = part;
      } else {
        acc[c] = mfma_fp8(bv, av, acc[c]);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][3] + tot[c][1];
  if (s == 1234.5f) sink[blockIdx.x * kThreads + threadIdx.x] = s;  // keeps the loop; never true for the data used
}

// The 32x32x64 shape of the same instruction family for comparison: each
// MFMA (131072 FLOP) makes a 32x32 float32 block from 32 rows x 64 K of each
// operand, two of them per 128-K block. Plain: kChains / 2 accumulators of
// 16 registers (as many output values per wave as the 16x16 loop's), each
// taking two MFMAs per iteration. PROMOTE: per 128-K block the two MFMAs are
// chained into a 16-register partial, and the previous block's partial is
// promoted (16 FMAs); kChains / 4 chains, each with its accumulator, its
// partial and its totals (48 registers, the footprint a GEMM wave has per
// 32x32 block it promotes), so that the loop needs no more registers than
// two waves per SIMD have.
template <bool PROMOTE>
__global__ void __launch_bounds__(kThreads, 1) mfma32_ceiling_kernel(const i32x4* frag, float* sink, int iters) {
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  constexpr int kC = PROMOTE ? kChains / 4 : kChains / 2;
  const int lane = threadIdx.x & 63;
  const i32x4 x0 = frag[lane], x1 = frag[64 + lane], y0 = frag[128 + lane], y1 = frag[192 + lane];
  const i32x8 a = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  const i32x8 b = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
  const float w = __builtin_bit_cast(float, 0x3f800000 | (lane & 7));
  f32x16 acc[kC], tot[kC];
#pragma unroll
  for (int c = 0; c < kC; ++c) acc[c] = tot[c] = (f32x16){};
  i32x8 av = a, bv = b;
  for (int it = 0; it < iters; ++it) {
    asm volatile("" : "+v"(av), "+v"(bv));
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      if constexpr (PROMOTE) {
        asm volatile("" : "+v"(av));
        f32x16 part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, (f32x16){}, 0, 0, 0, 0, 0, 0);
        part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, part, 0, 0, 0, 0, 0, 0);
        tot[c] += acc[c] * w;
        acc[c] = part;
      } else {
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, acc[c], 0, 0, 0, 0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[c], 0, 0, 0, 0, 0, 0);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kC; ++c) s += acc[c][0] + acc[c][15] + tot[c][1];
  if (s == 1234.5f) sink[blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace
}  // namespace dg

extern "C" dg_status dg_mfma_fp8_ceiling(const void* fragments, float* sink, int iters, int variant,
                                         long long* flops, void* stream) {
  if (!fragments || !sink || !flops) return DG_ERR_NULL;
  if (iters <= 0 || iters > (1 << 24) || variant < 0 || variant > 4) return DG_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(fragments) & 15u) != 0) return DG_ERR_ALIGN;
  const int cus = dg_get_num_cus();
  if (cus <= 0) return DG_ERR_DEVICE;
  void (*kern)(const dg::i32x4*, float*, int) =
      variant == 0 ? dg::mfma_ceiling_kernel<0>
    : variant == 1 ? dg::mfma_ceiling_kernel<1>
    : variant == 2 ? dg::mfma32_ceiling_kernel<false>
    : variant == 3 ? dg::mfma32_ceiling_kernel<true>
                   : dg::mfma_ceiling_kernel<2>;
  hipLaunchKernelGGL(kern, dim3(cus), dim3(dg::kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const dg::i32x4*>(fragments), sink, iters);
  if (hipGetLastError() != hipSuccess) return DG_ERR_LAUNCH;
  // Per wave and iteration, 16x16: kChains MFMAs of 2*16*16*128 FLOP;
  // 32x32: kChains / 2 (plain) or kChains / 4 (promoted) chains, two MFMAs
  // of 2*32*32*64 FLOP each.
  const long long per_iter = variant == 2 ? (dg::kChains / 2) * 2LL * 2 * 32 * 32 * 64
                           : variant == 3 ? (dg::kChains / 4) * 2LL * 2 * 32 * 32 * 64
                                          : dg::kChains * 2LL * 16 * 16 * 128;
  *flops = (long long)cus * (dg::kThreads / 64) * iters * per_iter;
  return DG_OK;
}
