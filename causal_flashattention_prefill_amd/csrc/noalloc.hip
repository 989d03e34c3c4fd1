// Device-side job table in a static buffer, for zyfa_fwd_noalloc: callers
// that cannot allocate device memory (graph capture without a prepared
// plan, tight serving loops, harnesses that forbid allocation).
//
// The plan cache of zyfa_fwd allocates a job table per shape and copies it
// from the host. Here the table is written by a small kernel, from the one
// definition in plan.h (job_entry), into `scratch`: a file-scope device
// array held on every GPU the library runs on until the process ends. Each
// call rewrites the table on its own stream just before the attention
// kernel reads it, so calls that overlap on one GPU race on it.
#include <mutex>

#include "device_common.h"
#include "plan.h"
#include "zyfa_internal.h"

namespace zyfa {

// 65536 job-table entries of 8 bytes: 512 KiB per GPU.
constexpr int kScratchEntries = 65536;
static __device__ __align__(256) int2 scratch[kScratchEntries];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int2* g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch` per device

__global__ __launch_bounds__(256) void build_jobs_kernel(int2* table, int entries, int num_wgs, long long njobs,
                                                         int pairs, int group) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i >= entries) return;
  const int r = i / num_wgs, w = i - r * num_wgs;
  const JobEntry e = job_entry(r, w, njobs, num_wgs, pairs, group);
  table[i] = int2{e.bh, e.tile};
}

}  // namespace

int noalloc_scratch_entries() { return kScratchEntries; }

// The device address of `scratch` on device dev (current), looked up once
// per device; host code passes this address, never the array's name.
hipError_t noalloc_scratch(int dev, int2** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<int2*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_build_jobs(int2* table, int rows, int num_wgs, long long njobs, int pairs, int group,
                             hipStream_t s) {
  const int entries = rows * num_wgs;
  if (entries <= 0 || entries > kScratchEntries) return hipErrorInvalidValue;
  hipLaunchKernelGGL(build_jobs_kernel, dim3((entries + 255) / 256), dim3(256), 0, s, table, entries, num_wgs, njobs,
                     pairs, group);
  return hipGetLastError();
}

}  // namespace zyfa
