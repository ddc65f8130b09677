// kernels.hip -- the kernel-per-op executor, the small helper kernels and the
// launch functions; the persistent kernel's variants are in kernels_m*.hip,
// the device code they share in kernels.h.
#include <mutex>

#include "kernels.h"

namespace mk {

__global__ void __launch_bounds__(kThreads)
    mk_phase_kernel(const DevPlan *__restrict__ dplan, CallArgs ca_in, int first) {
  __shared__ Smem sm;
  CP &d = *(CP *)dplan;
  const CallArgs ca = resolve_args(d, ca_in);
  if (tidx() == 0) sm.imisc[2] = 0;
  __syncthreads();
  const int pos = ((const AS4 int *)d.task_pos)[first + (int)blockIdx.x];
  const TD t = td_from_table(d.tasks, pos);
  WState ws;
  init_ws(ws);
  run_task_once(sm, d, ca, t, ws);
  vm_drain();  // LDS-DMA loads the compiler does not track complete before the wave ends
}

__global__ void mk_stage_kernel(int32_t *tok, int32_t *pos, int B, int slot,
                                const int32_t *tokens, int i, int start) {
  const int b = threadIdx.x + blockIdx.x * blockDim.x;
  if (b >= B) return;
  tok[b] = b == slot ? tokens[i] : 0;
  pos[b] = b == slot ? start + i : -1;
}

__global__ void mk_stage_chunk_kernel(int32_t *tok, int32_t *pos, int32_t *rows, int B,
                                      const int32_t *tokens, int cnt, int start, int row) {
  const int b = threadIdx.x + blockIdx.x * blockDim.x;
  if (b >= B) return;
  tok[b] = b < cnt ? tokens[b] : 0;
  pos[b] = b < cnt ? start + b : -1;
  rows[b] = row;
}

__global__ void mk_bump_kernel(uint32_t *p) {
  if (threadIdx.x == 0) {
    const uint32_t v = p[0] + 1u;
    p[0] = v ? v : 1u;
  }
}

__global__ void mk_zero_kernel(uint32_t *p, int n) {
  const int i = threadIdx.x + blockIdx.x * blockDim.x;
  if (i < n) p[i] = 0u;
}

// ---------------------------------------------------------------- launch --
hipError_t launch_persistent_m0(const DevPlan *d, const CallArgs &ca, int grid, hipStream_t s);
hipError_t launch_persistent_m1(const DevPlan *d, const CallArgs &ca, int grid, hipStream_t s);
hipError_t launch_persistent_m2(const DevPlan *d, const CallArgs &ca, int grid, hipStream_t s);

hipError_t launch_persistent(const DevPlan *d, const CallArgs &ca, int grid, int mode,
                             hipStream_t s) {
  return mode == 1   ? launch_persistent_m1(d, ca, grid, s)
         : mode == 2 ? launch_persistent_m2(d, ca, grid, s)
                     : launch_persistent_m0(d, ca, grid, s);
}

hipError_t launch_phase(const DevPlan *d, const CallArgs &ca, int first, int count,
                        hipStream_t s) {
  hipLaunchKernelGGL(mk_phase_kernel, dim3(count), dim3(kThreads), 0, s, d, ca, first);
  return hipGetLastError();
}

hipError_t launch_stage(int32_t *stage_tok, int32_t *stage_pos, int B, int slot,
                        const int32_t *tokens, int i, int start, hipStream_t s) {
  hipLaunchKernelGGL(mk_stage_kernel, dim3((B + 255) / 256), dim3(256), 0, s, stage_tok,
                     stage_pos, B, slot, tokens, i, start);
  return hipGetLastError();
}

hipError_t launch_stage_chunk(int32_t *stage_tok, int32_t *stage_pos, int32_t *stage_rows, int B,
                              const int32_t *tokens, int cnt, int start, int row, hipStream_t s) {
  hipLaunchKernelGGL(mk_stage_chunk_kernel, dim3((B + 255) / 256), dim3(256), 0, s, stage_tok,
                     stage_pos, stage_rows, B, tokens, cnt, start, row);
  return hipGetLastError();
}

hipError_t launch_bump_tag(uint32_t *p, hipStream_t s) {
  hipLaunchKernelGGL(mk_bump_kernel, dim3(1), dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t *p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(mk_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

int persistent_lds_bytes() { return (int)sizeof(Smem); }

// Device state of plans built without allocating (mk_build_plan_noalloc).
// Each device holds its own copy from module load until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: host
// code uses only the address hipGetSymbolAddress reports for the device.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[64];
}  // namespace

hipError_t static_scratch(int device, void **ptr) {
  *ptr = nullptr;
  if (device < 0 || device >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace mk

