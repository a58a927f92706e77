// Dynamic LDS limits of the kernels (host side).
#include <mutex>
#include <vector>

#include "hst_launch.h"

namespace hst {

namespace {
struct LdsLimit {
  const void* kern;
  int dev;
  size_t bytes;
};
std::mutex g_lds_mu;
std::vector<LdsLimit> g_lds;  // one entry per (kernel, device) raised so far
}  // namespace

hipError_t raise_lds_limit(const void* kern, size_t bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_lds_mu);
  LdsLimit* hit = nullptr;
  for (LdsLimit& x : g_lds)
    if (x.kern == kern && x.dev == dev) hit = &x;
  if (hit != nullptr && hit->bytes >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
  if (e != hipSuccess) return e;
  if (hit != nullptr) hit->bytes = bytes;
  else g_lds.push_back(LdsLimit{kern, dev, bytes});
  return hipSuccess;
}

}  // namespace hst
