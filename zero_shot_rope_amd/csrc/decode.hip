// decode.hip -- single-token Dynamic Bifocal RoPE decode for gfx950: split-K + LSE reduce.
//
// The new token's query sits at position p = L - 1 and attends keys 0..L-1 of a cache that
// holds keys rotated at their BASE absolute positions. G is recomputed from this step's L.
// Keys with p - j < w0 (the last w0 keys) are local and use the base score q~ . k~_j; older
// keys are remote and are moved to aliased positions by the correction rotation
// R(Delta_j) k~_j, built in registers from the cached base key, so the cache is never
// rewritten when G changes (review page, Method; gist.science summary, Methodologie
// section 2: correction rotation of the active query and cached keys, additive composition).
//
// Split kernel: one wave per (key chunk, KV head, batch). The wave streams 32-key blocks:
//   K rows load straight into MFMA A-operand registers (lane = key), are rotated in
//   registers, and S^T = K Q^T runs on v_mfma_f32_32x32x16_bf16 with the KV head's query
//   heads as columns; V is transposed through a small LDS tile for O^T = V^T P^T.
//   Local and remote contributions share one running max; the wave writes the partial
//   (max, sum, unnormalised output) of its chunk to the workspace.
// Reduce kernel: merges the partials of all chunks by log-sum-exp and writes bf16 o / lse.
#include "device_common.hpp"
#include "launch.hpp"

namespace bifocal {

template <int D>
struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  float* ws;
  int Hq, Hkv, L, cap;
  int w0, G;
  int n_splits, chunk;
  float scale_log2;
  uint32_t W[D / 2];
};

template <int D>
__global__ __launch_bounds__(64) void decode_split_kernel(const DecodeArgs<D> a) {
  constexpr int NC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int VP = 32 + 4;  // V^T pitch (bf16) for a 32-key block: 2 banks mod 32 per row
  __shared__ __align__(16) uint16_t s_vt[D * VP];
  __shared__ uint32_t s_w[D / 2];

  const int lane = threadIdx.x, h = lane >> 5, col = lane & 31;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int Hg = a.Hq / a.Hkv;
  const int L = a.L, p = L - 1, w0 = a.w0, G = a.G;

  for (int t = lane; t < D / 2; t += 64) s_w[t] = a.W[t];
  __syncthreads();

  // Query operands (B of S^T = K Q^T): column col = query head g*Hg + col (zero if col >= Hg).
  u32x4 qt[NC], qr[NC];
  {
    const uint16_t* src = a.q + ((size_t)b * a.Hq + (size_t)g * Hg + col) * D + 8 * h;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qt[c] = u32x4{0, 0, 0, 0};
      if (col < Hg) qt[c] = *reinterpret_cast<const u32x4*>(src + 16 * c);
    }
    const int dq = correction_offset(p, G);
#pragma unroll
    for (int c = 0; c < NC / 2; ++c) {
      u32x4 lo = qt[c], hi = qt[c + NC / 2];
      rotate8(lo, hi, dq, &s_w[16 * c + 8 * h]);
      qr[c] = lo;
      qr[c + NC / 2] = hi;
    }
  }

  const size_t row_stride = (size_t)a.Hkv * D;
  const uint16_t* kbase = a.kc + (size_t)b * a.cap * row_stride + (size_t)g * D;
  const uint16_t* vbase = a.vc + (size_t)b * a.cap * row_stride + (size_t)g * D;
  const int k_begin = split * a.chunk;
  const int k_end = min(L, k_begin + a.chunk);

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m_run = kNegBig, l_run = 0.f;

  for (int blk = k_begin; blk < k_end; blk += 32) {
    // ---- K block: lane (col, h) holds key blk+col, d = 16c + 8h .. +8 ----
    const int j = blk + col;
    u32x4 kreg[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kreg[c] = u32x4{0, 0, 0, 0};
      if (j < L) kreg[c] = *reinterpret_cast<const u32x4*>(kbase + (size_t)j * row_stride + 16 * c + 8 * h);
    }
    // ---- V block -> LDS transposed (units of 4 keys x 8 d) ----
#pragma unroll
    for (int rep = 0; rep < (8 * (D / 8)) / 64; ++rep) {
      const int u = lane + 64 * rep;
      const int kg = u / (D / 8), dg = u % (D / 8);
      u32x4 row[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jj = blk + 4 * kg + r;
        row[r] = u32x4{0, 0, 0, 0};
        if (jj < L) row[r] = *reinterpret_cast<const u32x4*>(vbase + (size_t)jj * row_stride + 8 * dg);
      }
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int w = dd >> 1;
        u32x2 out;
        if ((dd & 1) == 0) {
          out[0] = (row[0][w] & 0xffffu) | (row[1][w] << 16);
          out[1] = (row[2][w] & 0xffffu) | (row[3][w] << 16);
        } else {
          out[0] = (row[0][w] >> 16) | (row[1][w] & 0xffff0000u);
          out[1] = (row[2][w] >> 16) | (row[3][w] & 0xffff0000u);
        }
        *reinterpret_cast<u32x2*>(s_vt + (8 * dg + dd) * VP + 4 * kg) = out;
      }
    }

    // ---- scores ----
    const bool has_loc = (w0 > 0) && (p - (blk + 31) < w0);
    const bool has_rem = (p - blk) >= w0;
    f32x16 s = f32x16{};
    if (has_rem) {
      u32x4 kr[NC];
      const int dk = correction_offset(j < L ? j : 0, G);
#pragma unroll
      for (int c = 0; c < NC / 2; ++c) {
        u32x4 lo = kreg[c], hi = kreg[c + NC / 2];
        rotate8(lo, hi, dk, &s_w[16 * c + 8 * h]);
        kr[c] = lo;
        kr[c + NC / 2] = hi;
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) s = mfma32(kr[c], qr[c], s);
    }
    if (has_loc) {
      f32x16 t = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c) t = mfma32(kreg[c], qt[c], t);
      if (has_rem) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (p - (blk + c_row(r, h)) < w0) s[r] = t[r];
      } else {
        s = t;
      }
    }

    // ---- online softmax for this lane's column (query head) ----
    const bool tail = blk + 31 >= L;
    float mx = kNegBig;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = s[r] * a.scale_log2;
      if (tail && blk + c_row(r, h) >= L) x = kNegBig;
      s[r] = x;
      mx = fmaxf(mx, x);
    }
    mx = pair_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] *= alpha;
    float ps = 0.f;
    u32x4 pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = fast_exp2(s[r] - m_new);
      ps += s[r];
    }
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
      for (int w = 0; w < 4; ++w) pb[ch][w] = pack_bf16x2(s[8 * ch + 2 * w], s[8 * ch + 2 * w + 1]);
    l_run += ps;

    __syncthreads();  // V^T tile written
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        const uint16_t* vr = s_vt + (32 * db + col) * VP + 16 * ch + 4 * h;
        const u32x2 v0 = *reinterpret_cast<const u32x2*>(vr);
        const u32x2 v1 = *reinterpret_cast<const u32x2*>(vr + 8);
        o[db] = mfma32(u32x4{v0[0], v0[1], v1[0], v1[1]}, pb[ch], o[db]);
      }
    __syncthreads();  // before the next block overwrites the tile
  }

  const float l_tot = pair_sum(l_run);
  if (col < Hg) {
    const int head = g * Hg + col;
    float* dst = a.ws + (((size_t)b * a.Hq + head) * a.n_splits + split) * (D + 2);
    if (h == 0) {
      dst[0] = m_run;
      dst[1] = l_tot;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[2 + 32 * db + c_row(r, h)] = o[db][r];
  }
}

// One workgroup of 256 threads per (query head, batch): block max of the split maxima, per-split
// weights in LDS, then thread (part, d) accumulates splits part, part+P, ... for element d.
constexpr int kMaxSplits = 4096;

__device__ __forceinline__ float block_reduce(float x, float* red, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float y = __shfl_xor(x, off);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  if (lane == 0) red[wave] = x;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  __syncthreads();
  return r;
}

template <int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(const float* __restrict__ ws, uint16_t* __restrict__ o,
                                                            float* __restrict__ lse, int Hq, int n_splits) {
  constexpr int P = 256 / D;
  __shared__ float s_wt[kMaxSplits];
  __shared__ float s_red[4];
  __shared__ float s_acc[256];
  const int head = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const float* src = ws + ((size_t)b * Hq + head) * n_splits * (D + 2);
  float m = kNegBig;
  for (int s = t; s < n_splits; s += 256) m = fmaxf(m, src[(size_t)s * (D + 2)]);
  const float M = block_reduce(m, s_red, true);
  float den = 0.f;
  for (int s = t; s < n_splits; s += 256) {
    const float w = fast_exp2(src[(size_t)s * (D + 2)] - M);
    s_wt[s] = w;
    den += w * src[(size_t)s * (D + 2) + 1];
  }
  den = block_reduce(den, s_red, false);  // ends with a barrier: s_wt is complete
  const int d = t % D, part = t / D;
  float acc = 0.f;
#pragma unroll 8
  for (int s = part; s < n_splits; s += P) acc += s_wt[s] * src[(size_t)s * (D + 2) + 2 + d];
  s_acc[t] = acc;
  __syncthreads();
  if (t < D) {
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < P; ++q) tot += s_acc[q * D + t];
    o[((size_t)b * Hq + head) * D + t] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(tot / den));
    if (lse != nullptr && t == 0) lse[(size_t)b * Hq + head] = (M + __log2f(den)) * 0.69314718055994531f;
  }
}

DecodeSplit decode_split(long long L, int batch, int n_kv_heads) {
  // Aim for ~2048 waves in flight-sized grids (8 per CU on 256 CUs), 32-key granularity.
  const long long target = (2048 + (long long)batch * n_kv_heads - 1) / ((long long)batch * n_kv_heads);
  const long long blocks = (L + 31) / 32;
  long long ns = blocks < target ? blocks : target;
  if (ns < 1) ns = 1;
  long long chunk = (L + ns - 1) / ns;
  chunk = (chunk + 31) / 32 * 32;
  const long long bound = ns;  // monotone in L: the workspace is sized from this
  ns = (L + chunk - 1) / chunk;  // <= bound, since chunk >= L / bound
  return DecodeSplit{(int)ns, (int)chunk, (int)bound};
}

template <int D>
static hipError_t launch_decode_d(const DecodeLaunch& p, hipStream_t stream) {
  DecodeArgs<D> a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.kc = static_cast<const uint16_t*>(p.k_cache);
  a.vc = static_cast<const uint16_t*>(p.v_cache);
  a.ws = p.workspace;
  a.Hq = p.n_q_heads;
  a.Hkv = p.n_kv_heads;
  a.L = p.L;
  a.cap = p.capacity;
  a.w0 = p.w0;
  a.G = p.G;
  a.n_splits = p.n_splits;
  a.chunk = p.chunk;
  a.scale_log2 = p.scale_log2;
  for (int i = 0; i < D / 2; ++i) a.W[i] = p.W[i];
  hipLaunchKernelGGL(decode_split_kernel<D>, dim3(p.n_splits, p.n_kv_heads, p.batch), dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_reduce_kernel<D>, dim3(p.n_q_heads, p.batch), dim3(256), 0, stream,
                     (const float*)p.workspace, static_cast<uint16_t*>(p.o), p.lse, p.n_q_heads, p.n_splits);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeLaunch& p, hipStream_t stream) {
  if (p.head_dim == 128) return launch_decode_d<128>(p, stream);
  if (p.head_dim == 64) return launch_decode_d<64>(p, stream);
  return hipErrorInvalidValue;
}

// Parity hook: G and f(x) from the same device position helpers the attention kernels use.
__global__ void positions_kernel(int L, int G, int32_t* __restrict__ f_out, int32_t* __restrict__ G_out) {
  const int x = blockIdx.x * blockDim.x + threadIdx.x;
  if (x < L) f_out[x] = aliased_position(x, G);
  if (x == 0) G_out[0] = G;
}

hipError_t launch_positions(int L, int G, int32_t* f_out, int32_t* G_out, hipStream_t stream) {
  const int threads = 256;
  const int blocks = (L + threads - 1) / threads;
  hipLaunchKernelGGL(positions_kernel, dim3(blocks), dim3(threads), 0, stream, L, G, f_out, G_out);
  return hipGetLastError();
}

}  // namespace bifocal
