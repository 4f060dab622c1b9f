// Cross-entropy with ignore_index and z-loss, forward and backward in one call.
// Kernels and their definition: xent_kernels.hpp.
#include <mutex>

#include "xent_kernels.hpp"

using namespace fo;

extern "C" size_t fo_xent_workspace(int64_t T, int64_t V) {
  if (T < 0 || V < 1) return 0;
  return 256 + 2 * align_up((size_t)T * sizeof(float), 256);
}

namespace {

// compute units of the current device (one persistent row workgroup each)
int64_t cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return 256;
  return n;
}

template <typename T>
int xent_impl(const xent::RowArgs& a, const void* z, void* dz, float* loss, float* z_loss,
              int64_t* n_valid, int32_t* status, hipStream_t st) {
  if (a.T > 0) {
    xent::count_targets<<<1, 1024, 0, st>>>(a.T, a.V, a.tg, a.ignore,
                                            const_cast<xent::Counters*>(a.cnt));
    if (xent::launch_rows<T, T>(a, static_cast<const T*>(z), static_cast<T*>(dz), st,
                                cu_count()) != hipSuccess)
      return FO_ERR_HIP;
  } else {
    xent::count_targets<<<1, 1024, 0, st>>>(0, a.V, a.tg, a.ignore,
                                            const_cast<xent::Counters*>(a.cnt));
  }
  xent::finalize<<<1, 1024, 0, st>>>(a.T, a.row_loss, a.row_z, a.cnt, loss, z_loss, n_valid,
                                     status);
  return launch_status();
}

}  // namespace

namespace {

// The argument checks of both entry points, workspace aside.
int xent_check(int dtype, int64_t T, int64_t V, const void* logits, int64_t ldl,
               const int64_t* targets, const void* dlogits, int64_t ldd, const float* loss) {
  if (dtype != FO_F32 && dtype != FO_BF16) return FO_ERR_DTYPE;
  if (T < 0 || V < 1 || T > INT32_MAX) return FO_ERR_SHAPE;
  if (ldl < V || (dlogits != nullptr && ldd < V)) return FO_ERR_STRIDE;
  if (!loss) return FO_ERR_NULL;
  if (T > 0 && (!logits || !targets)) return FO_ERR_NULL;
  return FO_OK;
}

// Validates the arguments and runs the call with the workspace at w (ws_bytes of it).
int xent_call(int dtype, int64_t T, int64_t V, const void* logits, int64_t ldl,
              const int64_t* targets, int64_t ignore_index, float z_loss_coef, float dloss,
              void* dlogits, int64_t ldd, float* loss, float* z_loss, int64_t* n_valid,
              int32_t* status, char* w, size_t ws_bytes, void* stream) {
  const int rc = xent_check(dtype, T, V, logits, ldl, targets, dlogits, ldd, loss);
  if (rc != FO_OK) return rc;
  if (!w || ws_bytes < fo_xent_workspace(T, V)) return FO_ERR_WORKSPACE;
  xent::RowArgs a;
  a.T = T;
  a.V = V;
  a.ldz = ldl;
  a.ldd = ldd;
  a.ignore = ignore_index;
  a.zc = z_loss_coef;
  a.dloss = dloss;
  a.tg = targets;
  a.cnt = reinterpret_cast<const xent::Counters*>(w);
  a.row_loss = reinterpret_cast<float*>(w + 256);
  a.row_z = reinterpret_cast<float*>(w + 256 + align_up((size_t)T * sizeof(float), 256));
  hipStream_t st = as_stream(stream);
  return dtype == FO_F32
             ? xent_impl<float>(a, logits, dlogits, loss, z_loss, n_valid, status, st)
             : xent_impl<bf16>(a, logits, dlogits, loss, z_loss, n_valid, status, st);
}

// The no-allocation variant's workspace: one array per device (each GPU the library
// runs on holds its own copy until the process ends), sized for kNoAllocMaxT rows.
// Its name is only a host-side handle: kernels get the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
// Nothing in it has to start at zero: the counters and every row's loss terms are
// written before they are read, on every call.
constexpr int64_t kNoAllocMaxT = FO_XENT_NOALLOC_MAX_T;
constexpr size_t kScratchBytes = 256 + 2 * ((size_t)kNoAllocMaxT * sizeof(float));
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (FO_OK), or an error status.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FO_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return FO_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FO_OK;
}

}  // namespace

extern "C" int fo_xent_fwd_bwd(int dtype, int64_t T, int64_t V, const void* logits, int64_t ldl,
                               const int64_t* targets, int64_t ignore_index, float z_loss_coef,
                               float dloss, void* dlogits, int64_t ldd, float* loss,
                               float* z_loss, int64_t* n_valid, int32_t* status, void* ws,
                               size_t ws_bytes, void* stream) {
  return xent_call(dtype, T, V, logits, ldl, targets, ignore_index, z_loss_coef, dloss,
                   dlogits, ldd, loss, z_loss, n_valid, status, static_cast<char*>(ws),
                   ws_bytes, stream);
}

extern "C" int fo_xent_fwd_bwd_noalloc(int dtype, int64_t T, int64_t V, const void* logits,
                                       int64_t ldl, const int64_t* targets,
                                       int64_t ignore_index, float z_loss_coef, float dloss,
                                       void* dlogits, int64_t ldd, float* loss, float* z_loss,
                                       int64_t* n_valid, int32_t* status, void* stream) {
  int rc = xent_check(dtype, T, V, logits, ldl, targets, dlogits, ldd, loss);
  if (rc != FO_OK) return rc;
  if (T > kNoAllocMaxT) return FO_ERR_WORKSPACE;
  void* w = nullptr;
  rc = scratch_address(&w);
  if (rc != FO_OK) return rc;
  return xent_call(dtype, T, V, logits, ldl, targets, ignore_index, z_loss_coef, dloss,
                   dlogits, ldd, loss, z_loss, n_valid, status, static_cast<char*>(w),
                   kScratchBytes, stream);
}
