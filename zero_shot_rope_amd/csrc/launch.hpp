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
  float* o32 = nullptr;  // with local_only: O written here in fp32 (same layout) instead of to o
  float* lse;
  int batch, n_q_heads, n_kv_heads, head_dim;
  int L;       // keys 0..L-1; the query rows are positions L - Lq .. L - 1
  int Lq;      // query rows (L for a plain prefill)
  int kv_cap;  // rows per batch in k and v (L for a plain prefill, the capacity for a cache)
  int w0;  // clamped to [0, L]
  int G;
  float scale_log2;      // log2(e) / sqrt(head_dim)
  const uint32_t* W;     // head_dim / 2 fixed-point phase increments (host memory)
  bool local_only = false;  // one plain attention pass over the pairs 0 <= i - j < w0, no remote pass
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
  // Decode step on a raw new token (NULL otherwise): q is the raw query and k_new / v_new the raw
  // key and value of position L - 1, which the split kernel rotates and writes into cache row L - 1.
  const void* k_new = nullptr;
  const void* v_new = nullptr;
};

// Rows rotated by their correction offsets into a separate buffer: dst[b][r][h] =
// R(Delta_{pos0 + r}) src[b][r][h] for r < rows (src_cap / dst_cap rows per batch).
struct RotateRowsLaunch {
  const void* src;
  void* dst;
  int batch, rows, heads, head_dim;
  int src_cap, dst_cap, pos0, G;
  const uint32_t* W;
};

// Inclusion-exclusion merge of three attention passes: O_X [batch, rows, n_q_heads, head_dim]
// (bf16, or fp32 with f32_in), LSE_X [batch, n_q_heads, rows] fp32; has_window == false: passes
// A and C are empty.
struct Merge3Launch {
  const void* oa;
  const void* ob;
  const void* oc;
  const float* la;
  const float* lb;
  const float* lc;
  void* o;
  float* lse;
  int batch, rows, n_q_heads, head_dim;
  bool has_window;
  bool f32_in = false;
};

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream);
hipError_t launch_rotate_rows(const RotateRowsLaunch& p, hipStream_t stream);
hipError_t launch_merge3(const Merge3Launch& p, hipStream_t stream);
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
// Workgroups along x of a per-sequence-length decode (its workspace holds that many plus batch
// partial records).
long long decode_varlen_slots(int batch, int n_kv_heads);

// Static device scratch of bifocal_decode_noalloc (its size is the public maximum in bifocal.h).
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
// Address of the current device's scratch (looked up once per device, then cached).
hipError_t decode_scratch(float** out);

}  // namespace bifocal
