// Cross-entropy with ignore_index and z-loss, forward and backward in one call.
// Kernels and their definition: xent_kernels.hpp.
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

extern "C" int fo_xent_fwd_bwd(int dtype, int64_t T, int64_t V, const void* logits, int64_t ldl,
                               const int64_t* targets, int64_t ignore_index, float z_loss_coef,
                               float dloss, void* dlogits, int64_t ldd, float* loss,
                               float* z_loss, int64_t* n_valid, int32_t* status, void* ws,
                               size_t ws_bytes, void* stream) {
  if (dtype != FO_F32 && dtype != FO_BF16) return FO_ERR_DTYPE;
  if (T < 0 || V < 1 || T > INT32_MAX) return FO_ERR_SHAPE;
  if (ldl < V || (dlogits != nullptr && ldd < V)) return FO_ERR_STRIDE;
  if (!loss) return FO_ERR_NULL;
  if (T > 0 && (!logits || !targets)) return FO_ERR_NULL;
  if (!ws || ws_bytes < fo_xent_workspace(T, V)) return FO_ERR_WORKSPACE;
  char* w = static_cast<char*>(ws);
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
