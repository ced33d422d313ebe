// C ABI of the FP8 NT GEMM library: argument validation, CU-count setting and
// dispatch to the gfx950 kernels. The contract is documented in include/dg.h.

#include "../../include/dg.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "dg_internal.h"

namespace {

std::atomic<int> g_num_cus_override{0};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int tma_aligned(int x, int esize) { return (x + (16 / esize) - 1) / (16 / esize) * (16 / esize); }

// Per device: 0 = not yet queried, -1 = not a gfx950 (the kernels are built
// for it only), else the CU count. Filled once per device.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_cus[kMaxDevices];

int query_device_cus(int dev) {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return -1;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0 || (prop.gcnArchName[6] != '\0' && prop.gcnArchName[6] != ':'))
    return -1;
  return prop.multiProcessorCount > 0 ? prop.multiProcessorCount : -1;
}

// CU count of the current device, or 0 when there is none or it is not a
// gfx950.
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev >= kMaxDevices) {
    const int c = query_device_cus(dev);
    return c > 0 ? c : 0;
  }
  int c = g_device_cus[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    c = query_device_cus(dev);
    g_device_cus[dev].store(c, std::memory_order_relaxed);
  }
  return c > 0 ? c : 0;
}

int effective_cus() {
  const int dev_cus = device_cus();
  if (dev_cus <= 0) return 0;
  const int o = g_num_cus_override.load(std::memory_order_relaxed);
  return (o > 0 && o < dev_cus) ? o : dev_cus;
}

constexpr long long kMaxDim = 1 << 20;
constexpr long long kMaxBytes = 1LL << 40;
constexpr int kMaxMaskedGroups = dg::MAX_MASKED_GROUPS;
constexpr int kMaxNopadGroups = dg::MAX_NOPAD_GROUPS;

dg_status common_checks(const void* a, const float* sfa, const void* b, const float* sfb, const void* d,
                        long long n, long long k) {
  if (!a || !sfa || !b || !sfb || !d) return DG_ERR_NULL;
  if (n <= 0 || k <= 0 || n % 128 != 0 || k % 128 != 0) return DG_ERR_SHAPE;
  if (n > kMaxDim || k > kMaxDim) return DG_ERR_UNSUPPORTED;
  if (!aligned16(a) || !aligned16(b) || !aligned16(d) || !aligned16(sfa) || !aligned16(sfb)) return DG_ERR_ALIGN;
  return DG_OK;
}

dg_status launch(int kind, dg::GemmArgs& args, bool e8m0, void* stream) {
  args.scale_e8m0 = e8m0 ? 1 : 0;
  const int cus = effective_cus();
  if (cus <= 0) return DG_ERR_DEVICE;
  hipError_t e = dg::launch_gemm(kind, args, cus, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DG_OK : DG_ERR_LAUNCH;
}

dg_status dense(const void* a, const float* sfa, const void* b, const float* sfb, void* d, int m, int n, int k,
                bool e8m0, void* stream) {
  if (dg_status s = common_checks(a, sfa, b, sfb, d, n, k)) return s;
  if (m < 0) return DG_ERR_SHAPE;
  if ((long long)m * k >= kMaxBytes || (long long)m * n * 2 >= kMaxBytes || (long long)n * k >= kMaxBytes)
    return DG_ERR_UNSUPPORTED;
  if (m == 0) return DG_OK;
  dg::GemmArgs args{};
  args.a = static_cast<const uint8_t*>(a);
  args.sfa = sfa;
  args.b = static_cast<const uint8_t*>(b);
  args.sfb = sfb;
  args.d = static_cast<uint16_t*>(d);
  args.aux = nullptr;
  args.m = m;
  args.n = n;
  args.k = k;
  args.num_groups = 1;
  args.ld_sfa = tma_aligned(m, 4);
  return launch(dg::KIND_DENSE, args, e8m0, stream);
}

dg_status contiguous(const void* a, const float* sfa, const void* b, const float* sfb, void* d,
                     const int32_t* grouped_layout, int m, int n, int k, int num_groups, bool e8m0, void* stream) {
  if (dg_status s = common_checks(a, sfa, b, sfb, d, n, k)) return s;
  if (!grouped_layout) return DG_ERR_NULL;
  if (m < 0 || num_groups < 0 || m % 128 != 0) return DG_ERR_SHAPE;
  if ((long long)m * k >= kMaxBytes || (long long)m * n * 2 >= kMaxBytes ||
      (long long)num_groups * n * k >= kMaxBytes)
    return DG_ERR_UNSUPPORTED;
  if (m == 0 || num_groups == 0) return DG_OK;
  dg::GemmArgs args{};
  args.a = static_cast<const uint8_t*>(a);
  args.sfa = sfa;
  args.b = static_cast<const uint8_t*>(b);
  args.sfb = sfb;
  args.d = static_cast<uint16_t*>(d);
  args.aux = grouped_layout;
  args.m = m;
  args.n = n;
  args.k = k;
  args.num_groups = num_groups;
  args.ld_sfa = tma_aligned(m, 4);
  return launch(dg::KIND_CONTIGUOUS, args, e8m0, stream);
}

dg_status masked(const void* a, const float* sfa, const void* b, const float* sfb, void* d, const int32_t* masked_m,
                 int num_groups, int max_m, int n, int k, bool e8m0, void* stream) {
  if (dg_status s = common_checks(a, sfa, b, sfb, d, n, k)) return s;
  if (!masked_m) return DG_ERR_NULL;
  if (num_groups < 0 || max_m <= 0) return DG_ERR_SHAPE;
  if (num_groups > kMaxMaskedGroups) return DG_ERR_UNSUPPORTED;
  if ((long long)num_groups * max_m * k >= kMaxBytes || (long long)num_groups * max_m * n * 2 >= kMaxBytes ||
      (long long)num_groups * n * k >= kMaxBytes)
    return DG_ERR_UNSUPPORTED;
  if (num_groups == 0) return DG_OK;
  dg::GemmArgs args{};
  args.a = static_cast<const uint8_t*>(a);
  args.sfa = sfa;
  args.b = static_cast<const uint8_t*>(b);
  args.sfb = sfb;
  args.d = static_cast<uint16_t*>(d);
  args.aux = masked_m;
  args.m = max_m;
  args.n = n;
  args.k = k;
  args.num_groups = num_groups;
  args.ld_sfa = tma_aligned(max_m, 4);
  return launch(dg::KIND_MASKED, args, e8m0, stream);
}

dg_status nopad(const void* a, const float* sfa, const void* b, const float* sfb, void* d, const int32_t* group_rows,
                int m, int n, int k, int num_groups, bool e8m0, void* stream) {
  if (dg_status s = common_checks(a, sfa, b, sfb, d, n, k)) return s;
  if (!group_rows) return DG_ERR_NULL;
  if (m < 0 || num_groups < 0) return DG_ERR_SHAPE;
  if (num_groups > kMaxNopadGroups) return DG_ERR_UNSUPPORTED;
  if ((long long)m * k >= kMaxBytes || (long long)m * n * 2 >= kMaxBytes ||
      (long long)num_groups * n * k >= kMaxBytes)
    return DG_ERR_UNSUPPORTED;
  if (m == 0 || num_groups == 0) return DG_OK;
  dg::GemmArgs args{};
  args.a = static_cast<const uint8_t*>(a);
  args.sfa = sfa;
  args.b = static_cast<const uint8_t*>(b);
  args.sfb = sfb;
  args.d = static_cast<uint16_t*>(d);
  args.aux = group_rows;
  args.m = m;
  args.n = n;
  args.k = k;
  args.num_groups = num_groups;
  args.ld_sfa = tma_aligned(m, 4);
  return launch(dg::KIND_NOPAD, args, e8m0, stream);
}

}  // namespace

extern "C" {

dg_status dg_fp8_gemm_nt(const void* a, const float* sfa, const void* b, const float* sfb, void* d, int m, int n,
                         int k, void* stream) {
  return dense(a, sfa, b, sfb, d, m, n, k, false, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_contiguous(const void* a, const float* sfa, const void* b, const float* sfb,
                                              void* d, const int32_t* grouped_layout, int m, int n, int k,
                                              int num_groups, void* stream) {
  return contiguous(a, sfa, b, sfb, d, grouped_layout, m, n, k, num_groups, false, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_masked(const void* a, const float* sfa, const void* b, const float* sfb, void* d,
                                          const int32_t* masked_m, int num_groups, int max_m, int n, int k,
                                          void* stream) {
  return masked(a, sfa, b, sfb, d, masked_m, num_groups, max_m, n, k, false, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_nopad(const void* a, const float* sfa, const void* b, const float* sfb, void* d,
                                         const int32_t* group_rows, int m, int n, int k, int num_groups,
                                         void* stream) {
  return nopad(a, sfa, b, sfb, d, group_rows, m, n, k, num_groups, false, stream);
}

dg_status dg_fp8_gemm_nt_ue8m0(const void* a, const float* sfa, const void* b, const float* sfb, void* d, int m,
                               int n, int k, void* stream) {
  return dense(a, sfa, b, sfb, d, m, n, k, true, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const void* a, const float* sfa, const void* b,
                                                    const float* sfb, void* d, const int32_t* grouped_layout, int m,
                                                    int n, int k, int num_groups, void* stream) {
  return contiguous(a, sfa, b, sfb, d, grouped_layout, m, n, k, num_groups, true, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const void* a, const float* sfa, const void* b, const float* sfb,
                                                void* d, const int32_t* masked_m, int num_groups, int max_m, int n,
                                                int k, void* stream) {
  return masked(a, sfa, b, sfb, d, masked_m, num_groups, max_m, n, k, true, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_nopad_ue8m0(const void* a, const float* sfa, const void* b, const float* sfb,
                                               void* d, const int32_t* group_rows, int m, int n, int k,
                                               int num_groups, void* stream) {
  return nopad(a, sfa, b, sfb, d, group_rows, m, n, k, num_groups, true, stream);
}

dg_status dg_m_grouped_fp8_fp4_gemm_nt_contiguous(const void* a, const float* sfa, const void* b, const float* sfb,
                                                  void* d, const int32_t* grouped_layout, int m, int n, int k,
                                                  int num_groups, void* stream) {
  if (dg_status s = common_checks(a, sfa, b, sfb, d, n, k)) return s;
  if (!grouped_layout) return DG_ERR_NULL;
  if (m < 0 || num_groups < 0 || m % 128 != 0) return DG_ERR_SHAPE;
  if ((long long)m * k >= kMaxBytes || (long long)m * n * 2 >= kMaxBytes ||
      (long long)num_groups * n * (k / 2) >= kMaxBytes)
    return DG_ERR_UNSUPPORTED;
  if (m == 0 || num_groups == 0) return DG_OK;
  dg::GemmArgs args{};
  args.a = static_cast<const uint8_t*>(a);
  args.sfa = sfa;
  args.b = static_cast<const uint8_t*>(b);
  args.sfb = sfb;
  args.d = static_cast<uint16_t*>(d);
  args.aux = grouped_layout;
  args.m = m;
  args.n = n;
  args.k = k;
  args.num_groups = num_groups;
  args.ld_sfa = tma_aligned(m, 4);
  args.ld_sfb = tma_aligned(n, 4);
  args.scale_e8m0 = 1;
  const int cus = effective_cus();
  if (cus <= 0) return DG_ERR_DEVICE;
  return dg::launch_fp8_fp4(dg::KIND_CONTIGUOUS, args, cus, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? DG_OK
             : DG_ERR_LAUNCH;
}

dg_status dg_m_grouped_fp8_fp4_gemm_nt_masked(const void* a, const float* sfa, const void* b, const float* sfb,
                                              void* d, const int32_t* masked_m, int num_groups, int max_m, int n,
                                              int k, void* stream) {
  if (dg_status s = common_checks(a, sfa, b, sfb, d, n, k)) return s;
  if (!masked_m) return DG_ERR_NULL;
  if (num_groups < 0 || max_m <= 0) return DG_ERR_SHAPE;
  if (num_groups > kMaxMaskedGroups) return DG_ERR_UNSUPPORTED;
  if ((long long)num_groups * max_m * k >= kMaxBytes || (long long)num_groups * max_m * n * 2 >= kMaxBytes ||
      (long long)num_groups * n * (k / 2) >= kMaxBytes)
    return DG_ERR_UNSUPPORTED;
  if (num_groups == 0) return DG_OK;
  dg::GemmArgs args{};
  args.a = static_cast<const uint8_t*>(a);
  args.sfa = sfa;
  args.b = static_cast<const uint8_t*>(b);
  args.sfb = sfb;
  args.d = static_cast<uint16_t*>(d);
  args.aux = masked_m;
  args.m = max_m;
  args.n = n;
  args.k = k;
  args.num_groups = num_groups;
  args.ld_sfa = tma_aligned(max_m, 4);
  args.ld_sfb = tma_aligned(n, 4);
  args.scale_e8m0 = 1;
  const int cus = effective_cus();
  if (cus <= 0) return DG_ERR_DEVICE;
  return dg::launch_fp8_fp4(dg::KIND_MASKED, args, cus, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? DG_OK
             : DG_ERR_LAUNCH;
}

}  // extern "C"

namespace {

dg_status k_grouped(const void* a, const float* sfa, const void* b, const float* sfb, const float* c, float* d,
                    const int* ks, int num_groups, int m, int n, bool e8m0, void* stream) {
  if (!a || !sfa || !b || !sfb || !d || !ks) return DG_ERR_NULL;
  if (num_groups <= 0 || m < 0 || n <= 0 || n % 128 != 0) return DG_ERR_SHAPE;
  if (num_groups > dg::MAX_KGROUPED_GROUPS) return DG_ERR_UNSUPPORTED;
  if (n > kMaxDim) return DG_ERR_UNSUPPORTED;
  long long k = 0;
  for (int g = 0; g < num_groups; ++g) {
    if (ks[g] < 0 || ks[g] % 128 != 0) return DG_ERR_SHAPE;
    k += ks[g];
    if (k > kMaxDim) return DG_ERR_UNSUPPORTED;
  }
  if ((long long)m * k >= kMaxBytes || (long long)n * k >= kMaxBytes ||
      (long long)num_groups * m * n * 4 >= kMaxBytes)
    return DG_ERR_UNSUPPORTED;
  if (!aligned16(a) || !aligned16(b) || !aligned16(d) || !aligned16(sfa) || !aligned16(sfb) ||
      (c && !aligned16(c)))
    return DG_ERR_ALIGN;
  if (m == 0) return DG_OK;
  dg::KGroupedArgs args{};
  args.a = static_cast<const uint8_t*>(a);
  args.sfa = sfa;
  args.b = static_cast<const uint8_t*>(b);
  args.sfb = sfb;
  args.c = c;
  args.d = d;
  args.m = m;
  args.n = n;
  args.k = (int)k;
  args.num_groups = num_groups;
  args.ld_sfa = tma_aligned(m, 4);
  args.ld_sfb = tma_aligned(n, 4);
  args.scale_e8m0 = e8m0 ? 1 : 0;
  int off = 0;
  for (int g = 0; g < num_groups; ++g) {
    args.k_off[g] = off;
    off += ks[g] / 128;
  }
  args.k_off[num_groups] = off;
  const int cus = effective_cus();
  if (cus <= 0) return DG_ERR_DEVICE;
  return dg::launch_k_grouped(args, cus, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? DG_OK
                                                                                                : DG_ERR_LAUNCH;
}

}  // namespace

extern "C" {

dg_status dg_k_grouped_fp8_gemm_nt_contiguous(const void* a, const float* sfa, const void* b, const float* sfb,
                                              const float* c, float* d, const int* ks, int num_groups, int m, int n,
                                              void* stream) {
  return k_grouped(a, sfa, b, sfb, c, d, ks, num_groups, m, n, false, stream);
}

dg_status dg_k_grouped_fp8_gemm_nt_contiguous_ue8m0(const void* a, const float* sfa, const void* b,
                                                    const float* sfb, const float* c, float* d, const int* ks,
                                                    int num_groups, int m, int n, void* stream) {
  return k_grouped(a, sfa, b, sfb, c, d, ks, num_groups, m, n, true, stream);
}

int dg_get_mk_alignment_for_contiguous_layout(void) { return 128; }

int dg_get_tma_aligned_size(int x, int element_size) {
  if (x < 0 || element_size <= 0 || element_size > 16 || 16 % element_size != 0) return -1;
  return tma_aligned(x, element_size);
}

int dg_get_num_cus(void) { return effective_cus(); }

dg_status dg_set_num_cus(int num_cus) {
  g_num_cus_override.store(num_cus > 0 ? num_cus : 0, std::memory_order_relaxed);
  return DG_OK;
}

const char* dg_status_string(dg_status status) {
  switch (status) {
    case DG_OK: return "ok";
    case DG_ERR_NULL: return "null pointer argument";
    case DG_ERR_SHAPE: return "invalid shape (sizes must be non-negative; n, k multiples of 128; contiguous m a multiple of 128)";
    case DG_ERR_ALIGN: return "pointer not 16-byte aligned";
    case DG_ERR_UNSUPPORTED: return "size beyond the supported limits";
    case DG_ERR_LAUNCH: return "kernel launch failed";
    case DG_ERR_DEVICE: return "no usable HIP device";
    default: return "unknown status";
  }
}

}  // extern "C"
