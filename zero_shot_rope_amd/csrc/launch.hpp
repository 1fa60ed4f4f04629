// launch.hpp -- internal host-side launch descriptors (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bifocal {

// Arguments already validated by the C ABI layer; sizes fit in int.
struct PrefillLaunch {
  const void* q;
  const void* k;
  void* krot;  // NULL: fused in-kernel key rotation; else workspace for K' (prerotated mode)
  const void* v;
  void* o;
  float* lse;
  int batch, n_q_heads, n_kv_heads, head_dim;
  int L;       // keys 0..L-1; the query rows are positions L - Lq .. L - 1
  int Lq;      // query rows (L for a plain prefill)
  int kv_cap;  // rows per batch in k and v (L for a plain prefill, the capacity for a cache)
  int w0;  // clamped to [0, L]
  int G;
  float scale_log2;      // log2(e) / sqrt(head_dim)
  const uint32_t* W;     // head_dim / 2 fixed-point phase increments (host memory)
};

struct DecodeLaunch {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  void* o;
  float* lse;
  float* workspace;
  const int32_t* lens;  // per-sequence lengths on the device, or NULL (every sequence has length L)
  int batch, n_q_heads, n_kv_heads, head_dim;
  int L, capacity;  // with lens: L is the maximum length
  int w0;  // clamped to [0, L] (with lens: as requested; clamped per sequence on the device)
  int G;
  int w_pretrained;
  int n_splits, chunk;
  float scale_log2;
  const uint32_t* W;
};

// New token of a decode step: base RoPE at position p into q_out and cache row p, value copied.
struct RopeAppendLaunch {
  const void* q_raw;
  const void* k_raw;
  const void* v_new;
  void* q_out;
  void* k_cache;
  void* v_cache;
  int batch, n_q_heads, n_kv_heads, head_dim;
  int p, capacity;
  const uint32_t* W;
};

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream);
hipError_t launch_rope_append(const RopeAppendLaunch& r, hipStream_t stream);
hipError_t launch_decode(const DecodeLaunch& p, hipStream_t stream);
size_t prefill_workspace_bytes(long long batch, long long L, int n_kv_heads, int head_dim);
hipError_t launch_positions(int L, int G, int32_t* f_out, int32_t* G_out, hipStream_t stream);

// Decode split sizing shared by the workspace query and the launch.
struct DecodeSplit {
  int n_splits;
  int chunk;  // keys per split, a multiple of 32
  int max_splits;  // upper bound on n_splits for every length <= L (workspace sizing)
};
DecodeSplit decode_split(long long L, int batch, int n_kv_heads);

}  // namespace bifocal
