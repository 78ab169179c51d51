// qkv_create_static: a cache whose workspace is a device array of this file,
// for callers that cannot allocate device memory.
//
// `scratch` below is one file-scope device array; every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  In host
// code the array's name is only a host-side stand-in, so its device address
// is looked up once per device (with that device current) and kept; host code
// passes that address to the kernels (inside the cache's State) and never the
// array's name.  All caches created this way on one device share the array:
// creating another replaces the previous one, and calls on two such caches
// that overlap on one device race.
#include <hip/hip_runtime.h>

#include "qkv_internal.h"

namespace qkv {
int create_static_over(const qkv_config *cfg, void *workspace, size_t bytes, int dev, hipStream_t stream,
                       qkv_cache **out);
}

namespace {

constexpr size_t STATIC_BYTES = (size_t)QKV_STATIC_WORKSPACE_BYTES;
constexpr int MAX_DEVICES = 64;

static __device__ __align__(256) uint8_t scratch[STATIC_BYTES];

void *g_scratch_addr[MAX_DEVICES];   // device address of `scratch` per device (null: not looked up yet)

}  // namespace

extern "C" int qkv_create_static(const qkv_config *cfg, qkv_stream stream, qkv_cache **out) {
  if (!out) return QKV_EINVAL;
  *out = nullptr;
  if (qkv_check_config(cfg) != QKV_OK) return QKV_EINVAL;
  if (qkv_workspace_bytes(cfg) > STATIC_BYTES) return QKV_ECAPACITY;   // beyond the array: refused
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QKV_EHIP;
  if (dev < 0 || dev >= MAX_DEVICES) return QKV_EINVAL;
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QKV_EHIP;
    g_scratch_addr[dev] = p;
  }
  return qkv::create_static_over(cfg, g_scratch_addr[dev], STATIC_BYTES, dev, (hipStream_t)stream, out);
}
