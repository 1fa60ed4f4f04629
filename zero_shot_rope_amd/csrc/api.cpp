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

// The prefill kernels address a key/value tile row by a 32-bit byte offset (row < 64 times the
// row stride n_kv_heads * head_dim elements).
bool kv_row_fits(int n_kv_heads, int head_dim) { return (long long)n_kv_heads * head_dim < (1LL << 24); }

// Alignment the kernels' vector accesses assume: bf16 tensors and workspaces are read and
// written in 16-byte units, float and int32 arrays in 4-byte units. NULL passes both checks.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace of the unfused three-pass forms: the remote query and key copies, the three pass
// outputs (o_bytes per element: 4 for the prefill's fp32 outputs, 2 for the decode's bf16) and
// their LSEs, and (decode) the split workspace the passes share.
struct UnfusedLayout {
  size_t qrem, krem, o[3], l[3], dws, total;
};

UnfusedLayout unfused_layout(size_t q_rows, size_t k_rows, int n_q_heads, int n_kv_heads, int head_dim,
                             size_t lse_count, size_t dws_bytes, size_t o_bytes) {
  UnfusedLayout u;
  const size_t qb = align256(q_rows * n_q_heads * head_dim * 2);
  const size_t ob = align256(q_rows * n_q_heads * head_dim * o_bytes);
  const size_t kb = align256(k_rows * n_kv_heads * head_dim * 2);
  const size_t lb = align256(lse_count * 4);
  size_t at = 0;
  u.qrem = at;
  at += qb;
  u.krem = at;
  at += kb;
  for (int x = 0; x < 3; ++x) {
    u.o[x] = at;
    at += ob;
  }
  for (int x = 0; x < 3; ++x) {
    u.l[x] = at;
    at += lb;
  }
  u.dws = at;
  u.total = at + align256(dws_bytes);
  return u;
}

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
    case BIFOCAL_ESCRATCH: return "shapes need more than the static scratch of bifocal_decode_noalloc";
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
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(workspace) || !aligned4(lse))
    return BIFOCAL_EINVAL;
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1) return BIFOCAL_EINVAL;
  if (L < 1 || w0 < 0 || w_pretrained < 1 || !sane_theta(rope_theta)) return BIFOCAL_EINVAL;
  if (n_q_heads % n_kv_heads != 0) return BIFOCAL_EINVAL;
  if (!supported_head_dim(head_dim)) return BIFOCAL_EUNSUPPORTED;
  if (L > kMaxL || !kv_row_fits(n_kv_heads, head_dim)) return BIFOCAL_EUNSUPPORTED;
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
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || !aligned16(workspace) ||
      !aligned4(lse))
    return BIFOCAL_EINVAL;
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1) return BIFOCAL_EINVAL;
  if (q_len < 1 || q_offset < 0 || w0 < 0 || w_pretrained < 1 || !sane_theta(rope_theta)) return BIFOCAL_EINVAL;
  if (cache_capacity < 1 || q_offset > cache_capacity - q_len) return BIFOCAL_EINVAL;  // L <= capacity
  if (n_q_heads % n_kv_heads != 0) return BIFOCAL_EINVAL;
  if (!supported_head_dim(head_dim)) return BIFOCAL_EUNSUPPORTED;
  if (cache_capacity > kMaxL || !kv_row_fits(n_kv_heads, head_dim)) return BIFOCAL_EUNSUPPORTED;
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
  // One partial record (all query heads) per segment: a workgroup's run and a sequence meet in at
  // most workgroups + batch segments. Then a (first workgroup, count) pair per sequence.
  // Independent of the lengths, which only the device knows.
  const long long records = bifocal::decode_varlen_slots(batch, n_kv_heads) + batch;
  return static_cast<size_t>(records) * n_q_heads * (head_dim + 2) * sizeof(float) +
         static_cast<size_t>(batch) * 2 * sizeof(int32_t);
}

// Shared by the single-length and the per-sequence-length decode. lens == NULL: every sequence has
// length L; else lens is a device array and L the maximum length. Checks the shared arguments.
static int decode_impl(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int batch,
                       int n_q_heads, int n_kv_heads, int head_dim, const int32_t* lens, int64_t L,
                       int64_t cache_capacity, int64_t w0, int64_t w_pretrained, double rope_theta, void* workspace,
                       size_t workspace_bytes, void* stream, bool check_only = false,
                       const void* k_new = nullptr, const void* v_new = nullptr) {
  if (!q || !k_cache || !v_cache || !o) return BIFOCAL_EINVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || !aligned16(workspace) ||
      !aligned4(lse) || !aligned4(lens) || !aligned16(k_new) || !aligned16(v_new))
    return BIFOCAL_EINVAL;
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1) return BIFOCAL_EINVAL;
  if (L < 1 || cache_capacity < L || w0 < 0 || w_pretrained < 1 || !sane_theta(rope_theta))
    return BIFOCAL_EINVAL;
  if (n_q_heads % n_kv_heads != 0) return BIFOCAL_EINVAL;
  if (!supported_head_dim(head_dim)) return BIFOCAL_EUNSUPPORTED;
  // The query heads of one KV head are the 16 columns of the decode kernel's MFMA tile.
  if (n_q_heads / n_kv_heads > 16) return BIFOCAL_EUNSUPPORTED;
  if (cache_capacity > kMaxL || batch > 65535) return BIFOCAL_EUNSUPPORTED;  // grid z limit
  if (lens != nullptr && ((long double)bifocal::decode_varlen_slots(batch, n_kv_heads) + batch) * n_q_heads *
                               (head_dim + 2) * 4 >= 4.0e18L)
    return BIFOCAL_EUNSUPPORTED;  // workspace size beyond size_t arithmetic
  const size_t need = lens ? bifocal_decode_varlen_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, L)
                           : bifocal_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, L);
  if (!workspace || workspace_bytes < need) return BIFOCAL_EWORKSPACE;
  if (check_only) return BIFOCAL_OK;

  const int64_t G = bifocal_group_size(L, w_pretrained);
  uint32_t W[64];
  phase_increments(head_dim, rope_theta, W);
  // One length: the batch shares one grid of about one workgroup per CU. Per-sequence lengths:
  // the device lays the 32-key blocks of all sequences end to end and gives each of the
  // decode_varlen_slots workgroups an equal run of them.
  const bifocal::DecodeSplit s = bifocal::decode_split(L, batch, n_kv_heads);
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
  p.n_splits = lens ? static_cast<int>(bifocal::decode_varlen_slots(batch, n_kv_heads)) : s.n_splits;
  p.chunk = s.chunk;  // unused with per-sequence lengths
  p.scale_log2 = scale_log2_for(head_dim);
  p.W = W;
  p.k_new = k_new;
  p.v_new = v_new;
  return map_hip(bifocal::launch_decode(p, static_cast<hipStream_t>(stream)));
}

int bifocal_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                   int batch, int n_q_heads, int n_kv_heads, int head_dim,
                   int64_t L, int64_t cache_capacity, int64_t w0, int64_t w_pretrained,
                   double rope_theta, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, k_cache, v_cache, o, lse, batch, n_q_heads, n_kv_heads, head_dim, nullptr, L,
                     cache_capacity, w0, w_pretrained, rope_theta, workspace, workspace_bytes, stream);
}

int bifocal_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                           int batch, int n_q_heads, int n_kv_heads, int head_dim,
                           int64_t L, int64_t cache_capacity, int64_t w0, int64_t w_pretrained,
                           double rope_theta, void* stream) {
  // Every argument is checked before any HIP call (the workspace with a stand-in that is never
  // used), then the size this call needs against the static scratch.
  void* const stand_in = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
  const int st = decode_impl(q, k_cache, v_cache, o, lse, batch, n_q_heads, n_kv_heads, head_dim, nullptr, L,
                             cache_capacity, w0, w_pretrained, rope_theta, stand_in, ~static_cast<size_t>(0),
                             nullptr, /*check_only=*/true);
  if (st != BIFOCAL_OK) return st;
  const size_t need = bifocal_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, L);
  static_assert(bifocal::kDecodeScratchBytes == BIFOCAL_DECODE_NOALLOC_SCRATCH_BYTES, "scratch size mismatch");
  if (need == 0 || need > bifocal::kDecodeScratchBytes) return BIFOCAL_ESCRATCH;
  float* scratch = nullptr;
  if (bifocal::decode_scratch(&scratch) != hipSuccess) return BIFOCAL_EHIP;
  return decode_impl(q, k_cache, v_cache, o, lse, batch, n_q_heads, n_kv_heads, head_dim, nullptr, L,
                     cache_capacity, w0, w_pretrained, rope_theta, scratch, bifocal::kDecodeScratchBytes, stream);
}

size_t bifocal_prefill_unfused_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim, int64_t L) {
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || !supported_head_dim(head_dim) || L < 1 || L > kMaxL)
    return 0;
  const long double elems = (long double)batch * (long double)L * n_q_heads * head_dim;
  if (elems >= 1.0e17L) return 0;
  const size_t rows = static_cast<size_t>(batch) * static_cast<size_t>(L);
  return unfused_layout(rows, rows, n_q_heads, n_kv_heads, head_dim, rows * n_q_heads, 0, 4).total;
}

int bifocal_prefill_unfused(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                            int n_q_heads, int n_kv_heads, int head_dim, int64_t L, int64_t w0, int64_t w_pretrained,
                            double rope_theta, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o) return BIFOCAL_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(workspace) || !aligned4(lse))
    return BIFOCAL_EINVAL;
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1) return BIFOCAL_EINVAL;
  if (L < 1 || w0 < 0 || w_pretrained < 1 || !sane_theta(rope_theta)) return BIFOCAL_EINVAL;
  if (n_q_heads % n_kv_heads != 0) return BIFOCAL_EINVAL;
  if (!supported_head_dim(head_dim)) return BIFOCAL_EUNSUPPORTED;
  if (L > kMaxL || !kv_row_fits(n_kv_heads, head_dim)) return BIFOCAL_EUNSUPPORTED;
  const size_t need = bifocal_prefill_unfused_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, L);
  if (need == 0) return BIFOCAL_EUNSUPPORTED;
  if (!workspace || workspace_bytes < need) return BIFOCAL_EWORKSPACE;

  const size_t rows = static_cast<size_t>(batch) * static_cast<size_t>(L);
  const UnfusedLayout u = unfused_layout(rows, rows, n_q_heads, n_kv_heads, head_dim, rows * n_q_heads, 0, 4);
  char* ws = static_cast<char*>(workspace);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t G = bifocal_group_size(L, w_pretrained);
  const int w = static_cast<int>(w0 < L ? w0 : L);
  uint32_t W[64];
  phase_increments(head_dim, rope_theta, W);

  // Remote vectors q' = R(Delta_i) q~ and k' = R(Delta_j) k~, materialised.
  bifocal::RotateRowsLaunch r;
  r.batch = batch;
  r.rows = static_cast<int>(L);
  r.head_dim = head_dim;
  r.src_cap = r.dst_cap = static_cast<int>(L);
  r.pos0 = 0;
  r.G = static_cast<int>(G);
  r.W = W;
  r.src = q;
  r.dst = ws + u.qrem;
  r.heads = n_q_heads;
  int e = map_hip(bifocal::launch_rotate_rows(r, st));
  if (e != BIFOCAL_OK) return e;
  r.src = k;
  r.dst = ws + u.krem;
  r.heads = n_kv_heads;
  e = map_hip(bifocal::launch_rotate_rows(r, st));
  if (e != BIFOCAL_OK) return e;

  // Three plain attention passes: A (window, base), B (causal, remote), C (window, remote), each
  // writing its normalised output in fp32 so that the merge adds no bf16 rounding of its own.
  bifocal::PrefillLaunch p;
  p.krot = nullptr;
  p.v = v;
  p.batch = batch;
  p.n_q_heads = n_q_heads;
  p.n_kv_heads = n_kv_heads;
  p.head_dim = head_dim;
  p.L = p.Lq = p.kv_cap = static_cast<int>(L);
  p.G = 1;
  p.scale_log2 = scale_log2_for(head_dim);
  p.W = W;
  p.local_only = true;
  const void* pq[3] = {q, ws + u.qrem, ws + u.qrem};
  const void* pk[3] = {k, ws + u.krem, ws + u.krem};
  const int pw[3] = {w, static_cast<int>(L), w};
  for (int x = 0; x < 3; ++x) {
    if (pw[x] == 0) continue;  // w0 = 0: passes A and C hold no pair
    p.q = pq[x];
    p.k = pk[x];
    p.o = nullptr;
    p.o32 = reinterpret_cast<float*>(ws + u.o[x]);
    p.lse = reinterpret_cast<float*>(ws + u.l[x]);
    p.w0 = pw[x];
    e = map_hip(bifocal::launch_prefill(p, st));
    if (e != BIFOCAL_OK) return e;
  }

  bifocal::Merge3Launch m;
  m.oa = ws + u.o[0];
  m.ob = ws + u.o[1];
  m.oc = ws + u.o[2];
  m.la = reinterpret_cast<const float*>(ws + u.l[0]);
  m.lb = reinterpret_cast<const float*>(ws + u.l[1]);
  m.lc = reinterpret_cast<const float*>(ws + u.l[2]);
  m.o = o;
  m.lse = lse;
  m.batch = batch;
  m.rows = static_cast<int>(L);
  m.n_q_heads = n_q_heads;
  m.head_dim = head_dim;
  m.has_window = w > 0;
  m.f32_in = true;
  return map_hip(bifocal::launch_merge3(m, st));
}

size_t bifocal_decode_unfused_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                              int64_t cache_capacity) {
  const size_t dws = bifocal_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, cache_capacity);
  if (dws == 0 || cache_capacity > kMaxL) return 0;
  const size_t b = static_cast<size_t>(batch);
  return unfused_layout(b, b * static_cast<size_t>(cache_capacity), n_q_heads, n_kv_heads, head_dim,
                        b * n_q_heads, dws, 2).total;
}

int bifocal_decode_step(const void* q_raw, const void* k_raw, const void* v_new, void* k_cache, void* v_cache,
                        void* o, float* lse, int batch, int n_q_heads, int n_kv_heads, int head_dim,
                        int64_t L, int64_t cache_capacity, int64_t w0, int64_t w_pretrained, double rope_theta,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!q_raw || !k_raw || !v_new || !k_cache || !v_cache || !o) return BIFOCAL_EINVAL;
  // One launch pair: the split kernel of the chunk that ends at L applies base RoPE at L - 1 to
  // the query and the key and writes the key and the value into cache row L - 1.
  return decode_impl(q_raw, k_cache, v_cache, o, lse, batch, n_q_heads, n_kv_heads, head_dim, nullptr, L,
                     cache_capacity, w0, w_pretrained, rope_theta, workspace, workspace_bytes, stream, false, k_raw,
                     v_new);
}

int bifocal_decode_unfused(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int batch,
                           int n_q_heads, int n_kv_heads, int head_dim, int64_t L, int64_t cache_capacity, int64_t w0,
                           int64_t w_pretrained, double rope_theta, void* workspace, size_t workspace_bytes,
                           void* stream) {
  // Shapes and values are the decode's; the workspace is checked against this path's own size.
  const int st0 = decode_impl(q, k_cache, v_cache, o, lse, batch, n_q_heads, n_kv_heads, head_dim, nullptr, L,
                              cache_capacity, w0, w_pretrained, rope_theta, workspace, ~static_cast<size_t>(0),
                              nullptr, /*check_only=*/true);
  if (st0 != BIFOCAL_OK) return st0;
  const size_t need = bifocal_decode_unfused_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, cache_capacity);
  if (need == 0) return BIFOCAL_EUNSUPPORTED;
  if (workspace_bytes < need) return BIFOCAL_EWORKSPACE;

  const size_t b = static_cast<size_t>(batch);
  const size_t dws_bytes = bifocal_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, cache_capacity);
  const UnfusedLayout u = unfused_layout(b, b * static_cast<size_t>(cache_capacity), n_q_heads, n_kv_heads,
                                         head_dim, b * n_q_heads, dws_bytes, 2);
  char* ws = static_cast<char*>(workspace);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t G = bifocal_group_size(L, w_pretrained);
  const int64_t w = w0 < L ? w0 : L;
  uint32_t W[64];
  phase_increments(head_dim, rope_theta, W);

  // The whole cache's remote keys k' = R(Delta_j) k~ (j < L) into a copy with the cache's
  // layout, and the remote query q' = R(Delta_p) q~ at p = L - 1.
  bifocal::RotateRowsLaunch r;
  r.batch = batch;
  r.head_dim = head_dim;
  r.G = static_cast<int>(G);
  r.W = W;
  r.src = k_cache;
  r.dst = ws + u.krem;
  r.rows = static_cast<int>(L);
  r.heads = n_kv_heads;
  r.src_cap = r.dst_cap = static_cast<int>(cache_capacity);
  r.pos0 = 0;
  int e = map_hip(bifocal::launch_rotate_rows(r, st));
  if (e != BIFOCAL_OK) return e;
  r.src = q;
  r.dst = ws + u.qrem;
  r.rows = 1;
  r.heads = n_q_heads;
  r.src_cap = r.dst_cap = 1;
  r.pos0 = static_cast<int>(L - 1);
  e = map_hip(bifocal::launch_rotate_rows(r, st));
  if (e != BIFOCAL_OK) return e;

  // Three plain decode passes (G = 1, every pair local): A over the last w keys with base
  // vectors, B over all L keys with remote vectors, C over the last w keys with remote vectors.
  const size_t row_bytes = static_cast<size_t>(n_kv_heads) * head_dim * 2;
  const size_t win_off = static_cast<size_t>(L - w) * row_bytes;
  const char* kc = static_cast<const char*>(k_cache);
  const char* vc = static_cast<const char*>(v_cache);
  const char* kr = ws + u.krem;
  const void* pq[3] = {q, ws + u.qrem, ws + u.qrem};
  const void* pk[3] = {kc + win_off, kr, kr + win_off};
  const void* pv[3] = {vc + win_off, vc, vc + win_off};
  const int64_t pl[3] = {w, L, w};
  for (int x = 0; x < 3; ++x) {
    if (pl[x] == 0) continue;  // w0 = 0: passes A and C hold no pair
    e = decode_impl(pq[x], pk[x], pv[x], ws + u.o[x], reinterpret_cast<float*>(ws + u.l[x]), batch, n_q_heads,
                    n_kv_heads, head_dim, nullptr, pl[x], cache_capacity, pl[x], kMaxL, rope_theta, ws + u.dws,
                    dws_bytes, stream);
    if (e != BIFOCAL_OK) return e;
  }

  bifocal::Merge3Launch m;
  m.oa = ws + u.o[0];
  m.ob = ws + u.o[1];
  m.oc = ws + u.o[2];
  m.la = reinterpret_cast<const float*>(ws + u.l[0]);
  m.lb = reinterpret_cast<const float*>(ws + u.l[1]);
  m.lc = reinterpret_cast<const float*>(ws + u.l[2]);
  m.o = o;
  m.lse = lse;
  m.batch = batch;
  m.rows = 1;
  m.n_q_heads = n_q_heads;
  m.head_dim = head_dim;
  m.has_window = w > 0;
  return map_hip(bifocal::launch_merge3(m, st));
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
  if (!f_out || !G_out || !aligned4(f_out) || !aligned4(G_out)) return BIFOCAL_EINVAL;
  if (L < 1 || w_pretrained < 1 || L > 0x7fffffffLL) return BIFOCAL_EINVAL;
  const int64_t G = bifocal_group_size(L, w_pretrained);
  return map_hip(bifocal::launch_positions(static_cast<int>(L), static_cast<int>(G), f_out, G_out,
                                           static_cast<hipStream_t>(stream)));
}

}  // extern "C"
