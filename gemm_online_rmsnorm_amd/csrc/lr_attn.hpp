// Internal launch interface of the attention kernels (lr_attention.hip)
// for the C ABI (lr_api.cpp). Host-only declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lr {

// Causal RoPE attention, head dimension 128, bf16 (lr_attention.hip).
// Tensors are contiguous: Q, O, dO, dQ [T][H * 128]; K, V, dK, dV
// [T][Hkv * 128]; LSE and D [H][T] fp32. q and k are the rotated inputs.
struct AttnDesc {
  int T = 0, seq_len = 0, H = 0, Hkv = 0;
  double rope_base = 10000.0;
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  void* o = nullptr;
  const void* dout = nullptr;
  float* lse = nullptr;
  float* dsum = nullptr;
  float* lse2 = nullptr;
  void* dq = nullptr;
  void* dk = nullptr;
  void* dv = nullptr;
};
hipError_t run_rope(const void* x, void* y, int T, int heads, int seq_len, double rope_base,
                    bool inverse, hipStream_t s);
hipError_t run_attn_fwd(const AttnDesc& d, hipStream_t s);
hipError_t run_attn_dq(const AttnDesc& d, hipStream_t s);    // also writes d.dsum, d.lse2
hipError_t run_attn_dkdv(const AttnDesc& d, hipStream_t s);  // reads d.dsum, d.lse2

}  // namespace lr
