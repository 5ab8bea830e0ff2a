// Allocation-free variant of the optimizer step for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// muon_step_noalloc runs the same step as muon_step, but its workspace (the
// iterate, Gram and polynomial buffers, norm partials and descriptor table)
// is `scratch`, a static device array of this library: each GPU holds its own
// copy from the first use until the process ends.  The descriptor table is
// written into it by small kernels that carry the table bytes as kernel
// arguments, so the call needs no pinned staging memory either.
#include "../../include/muon.h"
#include "muon_common.h"

#include <mutex>

namespace muon {
int step_fixed_workspace(const muon_mat* params, const muon_mat* grads, muon_state* st,
                         const float* coeffs, int32_t steps, float lr, float wd, float beta,
                         void* stream, void* ws, size_t ws_bytes);
}  // namespace muon

namespace {

// One GPU's workspace for every allocation-free call on that GPU.
static __device__ __attribute__((aligned(256))) uint8_t scratch[MUON_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` per device, looked up once per device with that
// device current (the array's name is not a device address in host code).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MUON_E_HIP;
  if (dev >= kMaxDevices) return MUON_E_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MUON_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MUON_OK;
}

// Table bytes carried as kernel arguments (under the 4 KiB argument limit).
constexpr int kChunkWords = 960;
struct TableChunk {
  uint32_t* dst;
  uint32_t words;
  uint32_t _pad;
  uint32_t w[kChunkWords];
};

__global__ __launch_bounds__(256) void k_put_table(TableChunk c) {
  for (uint32_t i = threadIdx.x; i < c.words; i += blockDim.x) c.dst[i] = c.w[i];
}

}  // namespace

namespace muon {
hipError_t launch_put_table(void* dst, const uint8_t* bytes, size_t n, hipStream_t s) {
  if (n % 4 || reinterpret_cast<uintptr_t>(dst) % 4) return hipErrorInvalidValue;
  const size_t words = n / 4;
  for (size_t w0 = 0; w0 < words; w0 += kChunkWords) {
    TableChunk c;
    c.dst = static_cast<uint32_t*>(dst) + w0;
    c.words = static_cast<uint32_t>(words - w0 < size_t(kChunkWords) ? words - w0 : kChunkWords);
    c._pad = 0;
    __builtin_memcpy(c.w, bytes + 4 * w0, 4 * size_t(c.words));
    hipLaunchKernelGGL(k_put_table, dim3(1), dim3(256), 0, s, c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
}  // namespace muon

extern "C" int muon_step_noalloc(const muon_mat* params, const muon_mat* grads, muon_state* st,
                                 const float* coeffs, int32_t steps, float lr, float wd,
                                 float beta, void* stream) {
  void* ws = nullptr;
  const int rc = scratch_for_current_device(&ws);
  if (rc != MUON_OK) return rc;
  return muon::step_fixed_workspace(params, grads, st, coeffs, steps, lr, wd, beta, stream, ws,
                                    MUON_NOALLOC_SCRATCH_BYTES);
}
