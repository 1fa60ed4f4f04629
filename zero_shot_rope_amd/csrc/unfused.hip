// unfused.hip -- the unfused three-pass form of bifocal attention, kept as an ablation.
//
// The pages describe the prefill as three standard attention calls merged by inclusion-exclusion
// (review page, Method: passes A, B, C and the merge formula; gist.science summary, Methodologie
// section 2): A is sliding-window attention on the base-position vectors, B full causal
// attention on the remote (aliased) vectors, C sliding-window attention on the remote vectors,
// and O = (W_A O_A + W_B O_B - W_C O_C) / (W_A + W_B - W_C) with W_X = exp(LSE_X - M). Run that
// way, the remote vectors are materialised in memory first and every key is read three times.
// This file holds the two pieces the fused kernels do not have: a kernel that rotates rows of
// vectors by their correction offsets into a separate buffer, and the merge kernel. The three
// passes themselves are the all-local mode of the attention kernels on the right inputs.
#include "device_common.hpp"
#include "launch.hpp"

namespace bifocal {

template <int D>
struct RotateRowsArgs {
  uint32_t W[D / 2];
};

// dst[b][r][h] = R(Delta_{pos0 + r}) src[b][r][h] for rows r < Lr: one thread per 8 rotation
// pairs. src holds src_cap rows per batch and dst dst_cap rows per batch, H heads per row.
template <int D>
__global__ __launch_bounds__(256) void rotate_rows_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                          long long n_units, int H, int Lr, int src_cap, int dst_cap,
                                                          int pos0, int G, const RotateRowsArgs<D> a) {
  constexpr int HALF = D / 2, MCH = HALF / 8;
  const long long u = (long long)blockIdx.x * 256 + threadIdx.x;
  if (u >= n_units) return;
  const int m = (int)(u % MCH);
  const long long row = u / MCH;  // (b * Lr + r) * H + h
  const int h = (int)(row % H);
  const long long br = row / H;
  const int r = (int)(br % Lr);
  const long long b = br / Lr;
  const size_t s = ((size_t)(b * src_cap + r) * H + h) * D + 8 * m;
  const size_t d = ((size_t)(b * dst_cap + r) * H + h) * D + 8 * m;
  u32x4 lo = *reinterpret_cast<const u32x4*>(src + s);
  u32x4 hi = *reinterpret_cast<const u32x4*>(src + s + HALF);
  uint32_t w[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = a.W[8 * m + e];
  rotate8(lo, hi, correction_offset(pos0 + r, G), w);
  *reinterpret_cast<u32x4*>(dst + d) = lo;
  *reinterpret_cast<u32x4*>(dst + d + HALF) = hi;
}

// Inclusion-exclusion merge of the three passes. O_X [B, Lr, Hq, D] (T: uint16_t for bf16, float
// for fp32), LSE_X [B, Hq, Lr] fp32 (natural log). With has_window == 0 (w0 = 0) passes A and C have no pairs and are not read.
// One thread per 8 output elements; the weights are relative to M = max(LSE_A, LSE_B), which
// bounds all three (C's pairs are a subset of B's).
// Eight consecutive pass-output values as floats.
__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16lo(w[e]);
    x[2 * e + 1] = bf16hi(w[e]);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = a[e];
    x[4 + e] = b[e];
  }
}

template <int D, typename T>
__global__ __launch_bounds__(256) void merge3_kernel(const T* __restrict__ oa, const T* __restrict__ ob,
                                                     const T* __restrict__ oc, const float* __restrict__ la,
                                                     const float* __restrict__ lb, const float* __restrict__ lc,
                                                     uint16_t* __restrict__ o, float* __restrict__ lse,
                                                     long long n_units, int Lr, int Hq, int has_window) {
  constexpr int CH = D / 8;
  const long long u = (long long)blockIdx.x * 256 + threadIdx.x;
  if (u >= n_units) return;
  const int c = (int)(u % CH);
  const long long row = u / CH;  // (b * Lr + r) * Hq + h
  const int h = (int)(row % Hq);
  const long long br = row / Hq;
  const int r = (int)(br % Lr);
  const long long b = br / Lr;
  const size_t li = ((size_t)b * Hq + h) * Lr + r;
  const size_t oi = (size_t)row * D + 8 * c;
  const float lse_b = lb[li];
  const float lse_a = has_window ? la[li] : -INFINITY;
  const float lse_c = has_window ? lc[li] : -INFINITY;
  const float M = fmaxf(lse_a, lse_b);
  const float wa = has_window ? __expf(lse_a - M) : 0.f;
  const float wb = __expf(lse_b - M);
  const float wc = has_window ? __expf(lse_c - M) : 0.f;
  const float den = wa + wb - wc;
  const float inv = 1.0f / den;
  float xa[8] = {}, xb[8], xc[8] = {};
  load8(ob + oi, xb);
  if (has_window) {
    load8(oa + oi, xa);
    load8(oc + oi, xc);
  }
  u32x4 out;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float y0 = (wa * xa[2 * w] + wb * xb[2 * w] - wc * xc[2 * w]) * inv;
    const float y1 = (wa * xa[2 * w + 1] + wb * xb[2 * w + 1] - wc * xc[2 * w + 1]) * inv;
    out[w] = pack_bf16x2(y0, y1);
  }
  *reinterpret_cast<u32x4*>(o + oi) = out;
  if (lse != nullptr && c == 0) lse[li] = M + __logf(den);
}

template <int D>
static hipError_t launch_rotate_rows_d(const RotateRowsLaunch& p, hipStream_t stream) {
  RotateRowsArgs<D> a;
  for (int i = 0; i < D / 2; ++i) a.W[i] = p.W[i];
  const long long units = (long long)p.batch * p.rows * p.heads * (D / 16);
  if (units <= 0 || (units + 255) / 256 > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rotate_rows_kernel<D>, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(p.src), static_cast<uint16_t*>(p.dst), units, p.heads, p.rows,
                     p.src_cap, p.dst_cap, p.pos0, p.G, a);
  return hipGetLastError();
}

hipError_t launch_rotate_rows(const RotateRowsLaunch& p, hipStream_t stream) {
  if (p.head_dim == 128) return launch_rotate_rows_d<128>(p, stream);
  if (p.head_dim == 64) return launch_rotate_rows_d<64>(p, stream);
  return hipErrorInvalidValue;
}

template <int D, typename T>
static void merge3_d(const Merge3Launch& p, dim3 grid, long long units, hipStream_t stream) {
  hipLaunchKernelGGL((merge3_kernel<D, T>), grid, dim3(256), 0, stream, static_cast<const T*>(p.oa),
                     static_cast<const T*>(p.ob), static_cast<const T*>(p.oc), p.la, p.lb, p.lc,
                     static_cast<uint16_t*>(p.o), p.lse, units, p.rows, p.n_q_heads, p.has_window ? 1 : 0);
}

hipError_t launch_merge3(const Merge3Launch& p, hipStream_t stream) {
  const long long units = (long long)p.batch * p.rows * p.n_q_heads * (p.head_dim / 8);
  if (units <= 0 || (units + 255) / 256 > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((units + 255) / 256));
  if (p.head_dim == 128) {
    if (p.f32_in) merge3_d<128, float>(p, grid, units, stream);
    else merge3_d<128, uint16_t>(p, grid, units, stream);
  } else if (p.head_dim == 64) {
    if (p.f32_in) merge3_d<64, float>(p, grid, units, stream);
    else merge3_d<64, uint16_t>(p, grid, units, stream);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bifocal
