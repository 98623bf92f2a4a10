// kda_noalloc.hip -- kda_fwd_noalloc: kda_fwd_ex with its workspace in a fixed
// device array of the library instead of a caller buffer, for callers that cannot
// allocate device memory at all.
//
// The array is a file-scope __device__ variable, so every GPU the library runs on
// holds its own copy (KDA_NOALLOC_CAPACITY bytes) from the library's module load on
// that device until the process ends. Host code never passes the array's name to a
// kernel (in host code the name is only a host-side stand-in): once per device, with
// that device current, hipGetSymbolAddress gives the device copy's address, which is
// kept per device and handed to the kernels as their workspace pointer.
//
// Nothing in the array needs clearing between calls: within one call every word the
// kernels read is written first (the scheduler's tables, the intra-chunk records of
// every used chunk slot, the segment maps and states, a windowed call's carried state),
// so the previous call's contents never matter. All calls on one GPU share its array, so calls that overlap on one
// device (several streams, several host threads) race and must be serialised by the
// caller.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/kda.h"

namespace {

constexpr size_t CAPACITY = KDA_NOALLOC_CAPACITY;
static_assert(CAPACITY % 256 == 0, "capacity keeps the workspace alignment");

__device__ __align__(256) uint8_t scratch[CAPACITY];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_addr[MAX_DEVICES] = {};   // device address of each GPU's copy of the array, once looked up

// The device address of the current device's array (looked up once per device, with
// that device current); nullptr if the lookup fails.
void* scratch_address(int dev) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();   // leave no sticky error behind for the caller's next call
      return nullptr;
    }
    g_addr[dev] = p;
  }
  return g_addr[dev];
}

}  // namespace

extern "C" {

size_t kda_noalloc_capacity(void) { return CAPACITY; }

int kda_fwd_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
                    void* out, const float* A_log, const float* dt_bias, float lower_bound,
                    const void* initial_state, int initial_dtype, void* final_state, int final_dtype,
                    const int64_t* cu_seqlens, int64_t N, int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                    uint32_t flags, void* stream) {
  // sizes the workspace layout rejects, and every other argument error, are reported by
  // kda_fwd_ex itself, before anything is launched. A fixed-length call whose full
  // workspace exceeds the array runs in windows of chunk columns that fit it.
  const size_t need = kda_fwd_workspace_min(B, T, H, cu_seqlens ? N : 0);
  if (need > CAPACITY) return KDA_ERR_CAPACITY;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return KDA_ERR_HIP;
  void* ws = need > 0 ? scratch_address(dev) : nullptr;
  if (need > 0 && ws == nullptr) return KDA_ERR_HIP;
  return kda_fwd_ex(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state, initial_dtype,
                    final_state, final_dtype, cu_seqlens, N, B, T, H, K, V, flags, ws, ws ? CAPACITY : 0, stream);
}

}  // extern "C"
