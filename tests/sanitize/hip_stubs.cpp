// Host-only stand-ins for what fa_api.cpp calls outside itself: the kernel
// launchers of the other translation units and the two HIP runtime calls of
// its FA_DEBUG table checks.  They let the C-ABI layer be built and run with
// AddressSanitizer and UndefinedBehaviorSanitizer on a machine without a GPU.
// A launcher records the arguments it received and reports success; the HIP
// calls fail, so an FA_DEBUG path that reached them returns FA_ERR_HIP.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>

#include "fa_internal.h"

int g_launches = 0;
long long g_last_rows = 0;   // B * H * N of the last forward / merge launch

namespace fa {

hipError_t launch_fwd(const FwdArgs& a) {
  ++g_launches;
  if (a.B < 0 || a.H < 1 || a.N < 1 || (a.d != 64 && a.d != 128)) {
    std::fprintf(stderr, "launch_fwd reached with invalid sizes\n");
    std::abort();
  }
  g_last_rows = (long long)a.B * a.H * a.N;
  return hipSuccess;
}

hipError_t launch_merge(const MergeArgs& a) {
  ++g_launches;
  g_last_rows = a.rows;
  return hipSuccess;
}

hipError_t launch_bwd(const BwdArgs& a) {
  ++g_launches;
  if (a.Dvec == nullptr) std::abort();
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a) {
  ++g_launches;
  if (a.part == nullptr || a.num_seqs < 1) std::abort();
  return hipSuccess;
}

hipError_t launch_append(const AppendArgs& a) {
  ++g_launches;
  if (a.slot_map == nullptr || a.num_seqs < 1) std::abort();
  return hipSuccess;
}

hipError_t noalloc_scratch(void** ptr) {
  static unsigned char host_stand_in[256] __attribute__((aligned(256)));
  *ptr = host_stand_in;
  return hipSuccess;
}

}  // namespace fa

extern "C" {
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipErrorNoDevice; }
}
