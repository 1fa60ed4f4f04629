// api.cpp -- C ABI of the bifocal attention library (declared in include/bifocal.h).
//
// Host responsibilities: validate every argument before any HIP call, compute the group
// size G = max(1, ceil(L / w_pretrained)) in int64 (review page, Method; gist.science
// summary, Methodologie section 1), turn the RoPE frequencies theta^(-2k/D) into 0.32
// fixed-point phase increments in double precision, size the grids, launch on the
// caller's stream. No allocation, no host synchronisation, no state.
#include <math.h>
#include <stdint.h>

#include "../../include/bifocal.h"
#include "launch.hpp"

namespace {

constexpr long long kMaxL = 1LL << 30;

bool supported_head_dim(int d) { return d == 64 || d == 128; }

// W_k = round(2^32 * frac(omega_k / (2 pi))) mod 2^32, omega_k = theta^(-2k/D).
// frac() first, so that a frequency above one turn per step keeps its fractional part.
void phase_increments(int head_dim, double theta, uint32_t* W) {
  const double two_pi = 6.283185307179586476925286766559;
  for (int k = 0; k < head_dim / 2; ++k) {
    const double omega = pow(theta, -2.0 * k / head_dim);
    double turns = omega / two_pi;
    turns -= floor(turns);
    double fixed = nearbyint(turns * 4294967296.0);
    if (fixed >= 4294967296.0) fixed -= 4294967296.0;
    W[k] = static_cast<uint32_t>(fixed);
  }
}

float scale_log2_for(int head_dim) {
  return static_cast<float>(1.4426950408889634073599246810019 / sqrt(static_cast<double>(head_dim)));
}

int map_hip(hipError_t e) { return e == hipSuccess ? BIFOCAL_OK : BIFOCAL_EHIP; }

bool sane_theta(double t) { return t > 0.0 && isfinite(t); }

}  // namespace

extern "C" {

int64_t bifocal_group_size(int64_t L, int64_t w_pretrained) {
  if (L < 1 || w_pretrained < 1) return BIFOCAL_EINVAL;
  const int64_t g = L / w_pretrained + (L % w_pretrained != 0 ? 1 : 0);
  return g < 1 ? 1 : g;
}

const char* bifocal_status_string(int status) {
  switch (status) {
    case BIFOCAL_OK: return "ok";
    case BIFOCAL_EINVAL: return "invalid argument";
    case BIFOCAL_EUNSUPPORTED: return "unsupported configuration";
    case BIFOCAL_EWORKSPACE: return "workspace missing or too small";
    case BIFOCAL_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t bifocal_prefill_workspace_bytes(int batch, int n_kv_heads, int head_dim, int64_t L) {
  if (batch < 1 || n_kv_heads < 1 || !supported_head_dim(head_dim) || L < 1 || L > kMaxL) return 0;
  const long double bytes = (long double)batch * (long double)L * n_kv_heads * head_dim * 2;
  if (bytes >= 4.0e18L) return 0;
  return bifocal::prefill_workspace_bytes(batch, L, n_kv_heads, head_dim);
}

// Shared by the plain and the chunked prefill: query rows are positions L - Lq .. L - 1, keys
// 0 .. L - 1 are read from k/v with kv_cap rows per batch. Arguments already validated.
static int prefill_impl(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int n_q_heads,
                        int n_kv_heads, int head_dim, int64_t L, int64_t Lq, int64_t kv_cap, int64_t w0,
                        int64_t w_pretrained, double rope_theta, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (workspace != nullptr && workspace_bytes < bifocal_prefill_workspace_bytes(batch, n_kv_heads, head_dim, L))
    return BIFOCAL_EWORKSPACE;
  const int64_t G = bifocal_group_size(L, w_pretrained);
  uint32_t W[64];
  phase_increments(head_dim, rope_theta, W);
  bifocal::PrefillLaunch p;
  p.q = q;
  p.k = k;
  p.krot = workspace;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.batch = batch;
  p.n_q_heads = n_q_heads;
  p.n_kv_heads = n_kv_heads;
  p.head_dim = head_dim;
  p.L = static_cast<int>(L);
  p.Lq = static_cast<int>(Lq);
  p.kv_cap = static_cast<int>(kv_cap);
  // G == 1 makes the correction rotation the identity, so every pair scores as a local one:
  // run the all-local path (the base model exactly, with no rotation work).
  p.w0 = (G == 1 || w0 >= L) ? static_cast<int>(L) : static_cast<int>(w0);
  p.G = static_cast<int>(G);
  p.scale_log2 = scale_log2_for(head_dim);
  p.W = W;
  return map_hip(bifocal::launch_prefill(p, static_cast<hipStream_t>(stream)));
}

int bifocal_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                    int batch, int n_q_heads, int n_kv_heads, int head_dim,
                    int64_t L, int64_t w0, int64_t w_pretrained, double rope_theta,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o) return BIFOCAL_EINVAL;
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1) return BIFOCAL_EINVAL;
  if (L < 1 || w0 < 0 || w_pretrained < 1 || !sane_theta(rope_theta)) return BIFOCAL_EINVAL;
  if (n_q_heads % n_kv_heads != 0) return BIFOCAL_EINVAL;
  if (!supported_head_dim(head_dim)) return BIFOCAL_EUNSUPPORTED;
  if (L > kMaxL) return BIFOCAL_EUNSUPPORTED;
  const long double elems = (long double)batch * (long double)L * n_q_heads * head_dim;
  if (elems >= 4.0e18L) return BIFOCAL_EUNSUPPORTED;
  return prefill_impl(q, k, v, o, lse, batch, n_q_heads, n_kv_heads, head_dim, L, L, L, w0, w_pretrained,
                      rope_theta, workspace, workspace_bytes, stream);
}

int bifocal_prefill_chunk(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                          int batch, int n_q_heads, int n_kv_heads, int head_dim,
                          int64_t q_len, int64_t q_offset, int64_t cache_capacity,
                          int64_t w0, int64_t w_pretrained, double rope_theta,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !o) return BIFOCAL_EINVAL;
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1) return BIFOCAL_EINVAL;
  if (q_len < 1 || q_offset < 0 || w0 < 0 || w_pretrained < 1 || !sane_theta(rope_theta)) return BIFOCAL_EINVAL;
  if (cache_capacity < 1 || q_offset > cache_capacity - q_len) return BIFOCAL_EINVAL;  // L <= capacity
  if (n_q_heads % n_kv_heads != 0) return BIFOCAL_EINVAL;
  if (!supported_head_dim(head_dim)) return BIFOCAL_EUNSUPPORTED;
  if (cache_capacity > kMaxL) return BIFOCAL_EUNSUPPORTED;
  const long double elems = (long double)batch * (long double)cache_capacity * n_q_heads * head_dim;
  if (elems >= 4.0e18L) return BIFOCAL_EUNSUPPORTED;
  const int64_t L = q_offset + q_len;
  return prefill_impl(q, k_cache, v_cache, o, lse, batch, n_q_heads, n_kv_heads, head_dim, L, q_len,
                      cache_capacity, w0, w_pretrained, rope_theta, workspace, workspace_bytes, stream);
}

size_t bifocal_decode_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                      int64_t max_L) {
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1 || max_L < 1) return 0;
  if (max_L > kMaxL || n_q_heads % n_kv_heads != 0) return 0;
  const bifocal::DecodeSplit s = bifocal::decode_split(max_L, batch, n_kv_heads);
  return static_cast<size_t>(batch) * n_q_heads * s.max_splits * (head_dim + 2) * sizeof(float);
}

size_t bifocal_decode_varlen_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                             int64_t max_len) {
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1 || max_len < 1) return 0;
  if (max_len > kMaxL || n_q_heads % n_kv_heads != 0) return 0;
  const bifocal::DecodeSplit s = bifocal::decode_split(max_len, 1, n_kv_heads);
  return static_cast<size_t>(batch) * n_q_heads * s.max_splits * (head_dim + 2) * sizeof(float);
}

// Shared by the single-length and the per-sequence-length decode. lens == NULL: every sequence has
// length L; else lens is a device array and L the maximum length. Checks the shared arguments.
static int decode_impl(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int batch,
                       int n_q_heads, int n_kv_heads, int head_dim, const int32_t* lens, int64_t L,
                       int64_t cache_capacity, int64_t w0, int64_t w_pretrained, double rope_theta, void* workspace,
                       size_t workspace_bytes, void* stream, bool check_only = false) {
  if (!q || !k_cache || !v_cache || !o) return BIFOCAL_EINVAL;
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1) return BIFOCAL_EINVAL;
  if (L < 1 || cache_capacity < L || w0 < 0 || w_pretrained < 1 || !sane_theta(rope_theta))
    return BIFOCAL_EINVAL;
  if (n_q_heads % n_kv_heads != 0) return BIFOCAL_EINVAL;
  if (!supported_head_dim(head_dim)) return BIFOCAL_EUNSUPPORTED;
  const int group = n_q_heads / n_kv_heads;
  if (group != 1 && group != 2 && group != 4) return BIFOCAL_EUNSUPPORTED;
  if (cache_capacity > kMaxL || batch > 65535) return BIFOCAL_EUNSUPPORTED;  // grid z limit
  if (lens != nullptr && (long long)batch * bifocal::decode_split(L, 1, n_kv_heads).max_splits > 0x7fffffffLL)
    return BIFOCAL_EUNSUPPORTED;  // grid x limit of the interleaved per-sequence grid
  const size_t need = lens ? bifocal_decode_varlen_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, L)
                           : bifocal_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, L);
  if (!workspace || workspace_bytes < need) return BIFOCAL_EWORKSPACE;
  if (check_only) return BIFOCAL_OK;

  const int64_t G = bifocal_group_size(L, w_pretrained);
  uint32_t W[64];
  phase_increments(head_dim, rope_theta, W);
  // One length: the batch shares one grid of about one workgroup per CU. Per-sequence lengths:
  // each sequence is split as if it were alone (its chunks exist up to its own length).
  const bifocal::DecodeSplit s = bifocal::decode_split(L, lens ? 1 : batch, n_kv_heads);
  bifocal::DecodeLaunch p;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.o = o;
  p.lse = lse;
  p.workspace = static_cast<float*>(workspace);
  p.lens = lens;
  p.batch = batch;
  p.n_q_heads = n_q_heads;
  p.n_kv_heads = n_kv_heads;
  p.head_dim = head_dim;
  p.L = static_cast<int>(L);
  p.capacity = static_cast<int>(cache_capacity);
  if (lens == nullptr) p.w0 = (G == 1 || w0 >= L) ? static_cast<int>(L) : static_cast<int>(w0);
  else p.w0 = static_cast<int>(w0 < L ? w0 : L);  // clamped per sequence on the device
  p.G = static_cast<int>(G);
  p.w_pretrained = static_cast<int>(w_pretrained < (1LL << 30) ? w_pretrained : (1LL << 30));
  p.n_splits = s.n_splits;
  p.chunk = s.chunk;
  p.scale_log2 = scale_log2_for(head_dim);
  p.W = W;
  return map_hip(bifocal::launch_decode(p, static_cast<hipStream_t>(stream)));
}

int bifocal_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                   int batch, int n_q_heads, int n_kv_heads, int head_dim,
                   int64_t L, int64_t cache_capacity, int64_t w0, int64_t w_pretrained,
                   double rope_theta, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, k_cache, v_cache, o, lse, batch, n_q_heads, n_kv_heads, head_dim, nullptr, L,
                     cache_capacity, w0, w_pretrained, rope_theta, workspace, workspace_bytes, stream);
}

int bifocal_decode_step(const void* q_raw, const void* k_raw, const void* v_new, void* k_cache, void* v_cache,
                        void* o, float* lse, int batch, int n_q_heads, int n_kv_heads, int head_dim,
                        int64_t L, int64_t cache_capacity, int64_t w0, int64_t w_pretrained, double rope_theta,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!q_raw || !k_raw || !v_new || !k_cache || !v_cache || !o) return BIFOCAL_EINVAL;
  // All other checks are the decode's; run them before anything is written.
  const int st = decode_impl(o, k_cache, v_cache, o, lse, batch, n_q_heads, n_kv_heads, head_dim, nullptr, L,
                             cache_capacity, w0, w_pretrained, rope_theta, workspace, workspace_bytes, nullptr,
                             /*check_only=*/true);
  if (st != BIFOCAL_OK) return st;
  if ((long long)batch * (n_q_heads + n_kv_heads) * (head_dim / 16) > 0x7fffffffLL * 256)
    return BIFOCAL_EUNSUPPORTED;  // grid x limit of the new-token kernel
  uint32_t W[64];
  phase_increments(head_dim, rope_theta, W);
  bifocal::RopeAppendLaunch r;
  r.q_raw = q_raw;
  r.k_raw = k_raw;
  r.v_new = v_new;
  r.q_out = o;
  r.k_cache = k_cache;
  r.v_cache = v_cache;
  r.batch = batch;
  r.n_q_heads = n_q_heads;
  r.n_kv_heads = n_kv_heads;
  r.head_dim = head_dim;
  r.p = static_cast<int>(L - 1);
  r.capacity = static_cast<int>(cache_capacity);
  r.W = W;
  const int st2 = map_hip(bifocal::launch_rope_append(r, static_cast<hipStream_t>(stream)));
  if (st2 != BIFOCAL_OK) return st2;
  // The rotated query sits in o; the reduce overwrites it only after the split kernel read it.
  return decode_impl(o, k_cache, v_cache, o, lse, batch, n_q_heads, n_kv_heads, head_dim, nullptr, L,
                     cache_capacity, w0, w_pretrained, rope_theta, workspace, workspace_bytes, stream, false);
}

int bifocal_decode_varlen(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                          int batch, int n_q_heads, int n_kv_heads, int head_dim,
                          const int32_t* seq_lens, int64_t max_len, int64_t cache_capacity,
                          int64_t w0, int64_t w_pretrained, double rope_theta,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!seq_lens) return BIFOCAL_EINVAL;
  return decode_impl(q, k_cache, v_cache, o, lse, batch, n_q_heads, n_kv_heads, head_dim, seq_lens, max_len,
                     cache_capacity, w0, w_pretrained, rope_theta, workspace, workspace_bytes, stream);
}

int bifocal_positions(int64_t L, int64_t w_pretrained, int32_t* f_out, int32_t* G_out, void* stream) {
  if (!f_out || !G_out) return BIFOCAL_EINVAL;
  if (L < 1 || w_pretrained < 1 || L > 0x7fffffffLL) return BIFOCAL_EINVAL;
  const int64_t G = bifocal_group_size(L, w_pretrained);
  return map_hip(bifocal::launch_positions(static_cast<int>(L), static_cast<int>(G), f_out, G_out,
                                           static_cast<hipStream_t>(stream)));
}

}  // extern "C"
