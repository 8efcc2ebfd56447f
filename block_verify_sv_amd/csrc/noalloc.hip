// sv_verify_attention_noalloc: the verify-attention call for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// It runs exactly the kernels of sv_verify_attention, with the split-KV partials in a
// fixed scratch array that lives in this code object (one copy per GPU, 32 MiB, held
// until the process ends) instead of a caller-supplied workspace.  The array's host-side
// name is only a stand-in: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and that address is what the kernels
// receive.  Nothing is allocated, freed or cleared here; the attention kernels need no
// initial scratch contents.  Every call on one GPU shares that GPU's array, so calls
// that overlap in time on one GPU (different streams, or several host threads) race.
#include <hip/hip_runtime.h>
#include <stdio.h>

#include <mutex>

#include "internal.hpp"
#include "specverify.h"

namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(SV_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, once looked up

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

extern "C" sv_status sv_verify_attention_noalloc(const sv_attn_desc* desc, const void* q,
                                                 const void* k_cache, const void* v_cache,
                                                 const int32_t* page_table,
                                                 const int32_t* ctx_lens,
                                                 const uint64_t* block_mask, void* out,
                                                 float* lse, void* stream) {
  char msg[256];
  size_t need = 0;
  sv_status st = sv_verify_attention_workspace(desc, &need);
  if (st != SV_OK) return st;
  if (need > kScratchBytes) {
    snprintf(msg, sizeof msg,
             "this descriptor needs %zu bytes of split-KV scratch, more than the %zu bytes "
             "the allocation-free call holds; use sv_verify_attention with a workspace",
             need, kScratchBytes);
    return sv::report(SV_ERR_WORKSPACE, msg);
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    snprintf(msg, sizeof msg, "hipGetDevice: %s", hipGetErrorString(e));
    return sv::report(SV_ERR_DEVICE, msg);
  }
  if (dev < 0 || dev >= kMaxDevices)
    return sv::report(SV_ERR_UNSUPPORTED, "device ordinal beyond 63");
  if (stream) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) {
      snprintf(msg, sizeof msg, "hipStreamGetDevice: %s", hipGetErrorString(e));
      return sv::report(SV_ERR_DEVICE, msg);
    }
    if (static_cast<int>(sdev) != dev)
      return sv::report(SV_ERR_INVALID_ARG, "stream belongs to another device than the current one");
  }
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) {
        snprintf(msg, sizeof msg, "hipGetSymbolAddress(scratch): %s",
                 e != hipSuccess ? hipGetErrorString(e) : "null address");
        return sv::report(SV_ERR_DEVICE, msg);
      }
      g_scratch_ptr[dev] = p;
    }
    ptr = g_scratch_ptr[dev];
  }
  return sv::attention_call(desc, q, k_cache, v_cache, page_table, ctx_lens, block_mask, out, lse,
                            ptr, kScratchBytes, stream, "sv_verify_attention_noalloc launch");
}
