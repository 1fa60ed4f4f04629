// Split kernel: one workgroup of 8 waves per (key chunk, group of 8 KV heads, batch); wave w
//   owns KV head 8*blockIdx.y + w and walks the chunk in 32-key blocks. The 8 waves read the
//   same keys, so the workgroup streams each position's contiguous 2 KB of K and of V.
//   K rows load straight into MFMA A-operand registers (lane = key) and are rotated in
//   registers; V goes global->LDS by direct loads into a per-wave swizzled tile and is read
//   back transposed for O^T = V^T P^T. Each wave keeps the next block's K and V loads in
//   flight while it computes the current block (decode is a pure HBM stream; this keeps
//   ~128 KB per CU outstanding). S^T = K Q^T runs on v_mfma_f32_32x32x16_bf16 with the KV
//   head's query heads as columns. Local and remote contributions share one running max; the
//   wave writes the partial (max, sum, unnormalised output) of its chunk to the workspace.
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

constexpr int kDecWaves = 8;
constexpr int kDecBlock = 32;  // keys per block

template <int D>
__global__ __launch_bounds__(64 * kDecWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_split_kernel(const DecodeArgs<D> a) {
  constexpr int NC = D / 16, NDB = D / 32, CPR = D / 8, RPI = 64 / CPR;
  constexpr int VSZ = kDecBlock * D;       // elements of one wave's V tile
  constexpr int NLD = kDecBlock / RPI;     // direct loads per V tile
  // Separate objects per buffer so reads of one do not wait for direct loads into the other.
  __shared__ __align__(16) uint16_t s_v0[kDecWaves * VSZ], s_v1[kDecWaves * VSZ];
  __shared__ __align__(16) uint32_t s_w[D / 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int split = blockIdx.x, b = blockIdx.z;
  const int g = blockIdx.y * kDecWaves + wave;  // KV head of this wave
  const int Hg = a.Hq / a.Hkv;
  const int L = a.L, p = L - 1, w0 = a.w0, G = a.G;

  for (int t = tid; t < D / 2; t += 64 * kDecWaves) s_w[t] = a.W[t];
  __syncthreads();  // the only workgroup barrier: waves are independent from here on
  if (g >= a.Hkv) return;

  // Query operands (B of S^T = K Q^T): column col = query head g*Hg + col (zero if col >= Hg),
  // scaled into log2 units. qr = R(Delta_p) q~ stays in registers; q~ itself is only needed for
  // the blocks holding the last w0 keys and is re-read there.
  const uint16_t* qsrc = a.q + ((size_t)b * a.Hq + (size_t)g * Hg + col) * D + 8 * h;
  auto load_q = [&](u32x4 (&raw)[NC]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      raw[c] = u32x4{0, 0, 0, 0};
      if (col < Hg) raw[c] = *reinterpret_cast<const u32x4*>(qsrc + 16 * c);
    }
  };
  u32x4 qr[NC];
  {
    u32x4 raw[NC];
    load_q(raw);
    const int dq = correction_offset(p, G);
#pragma unroll
    for (int c = 0; c < NC / 2; ++c) {
      u32x4 lo = raw[c], hi = raw[c + NC / 2];
      rotate8_scaled(lo, hi, dq, &s_w[16 * c + 8 * h], a.scale_log2);
      qr[c] = lo;
      qr[c + NC / 2] = hi;
    }
  }

  const size_t row_stride = (size_t)a.Hkv * D;
  const uint16_t* kbase = a.kc + (size_t)b * a.cap * row_stride + (size_t)g * D;
  const uint16_t* vbase = a.vc + (size_t)b * a.cap * row_stride + (size_t)g * D;
  const int k_begin = split * a.chunk;
  const int k_end = min(L, k_begin + a.chunk);
  const int nblk = (k_end - k_begin + kDecBlock - 1) / kDecBlock;
  uint16_t* vb0 = s_v0 + wave * VSZ;
  uint16_t* vb1 = s_v1 + wave * VSZ;

  // K block: lane (col, h) holds key blk+col, d = 16c + 8h .. +8 (rows past L clamped to L-1;
  // their scores are masked).
  auto load_k = [&](int blk, u32x4 (&kr)[NC]) __attribute__((always_inline)) {
    const int j = min(blk + col, L - 1);
    const uint16_t* src = kbase + (size_t)j * row_stride + 8 * h;
#pragma unroll
    for (int c = 0; c < NC; ++c) kr[c] = *reinterpret_cast<const u32x4*>(src + 16 * c);
  };
  // V block -> this wave's LDS tile: load n fills rows RPI*n + lane/CPR, slot lane%CPR holding
  // global chunk slot ^ swz(row).
  auto load_v = [&](int blk, uint16_t* vb) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int row = RPI * n + lane / CPR;
      const int j = min(blk + row, L - 1);
      load_lds16(vbase + (size_t)j * row_stride + 8 * ((lane % CPR) ^ swz<D>(row)), vb + RPI * n * D);
    }
  };

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m_run = kNegBig, l_run = 0.f;
  const int tr_r = lane & 15;
  const int tr_key = 4 * h + (tr_r >> 2);
  const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (tr_r & 3);

  // `after_scores` runs once the K registers have been consumed (it reloads them for the
  // next block, so the K loads overlap this block's softmax and PV).
  auto compute = [&](int blk, u32x4 (&kr)[NC], const uint16_t* vb, auto after_scores) __attribute__((always_inline)) {
    // Keys blk .. blk+31: local iff p - j < w0 (the last w0 keys), else remote.
    const bool has_loc = (w0 > 0) && (p - (blk + kDecBlock - 1) < w0);
    const bool has_rem = (p - blk) >= w0;
    f32x16 s = f32x16{};
    if (has_loc) {
      u32x4 qt[NC];
      load_q(qt);
#pragma unroll
      for (int c = 0; c < NC; ++c) s = mfma32(kr[c], scale8(qt[c], a.scale_log2), s);
    }
    if (has_rem) {
      // Correction rotation R(Delta_j) of this lane's key, in place.
      const int dk = correction_offset(min(blk + col, L - 1), G);
#pragma unroll
      for (int c = 0; c < NC / 2; ++c) rotate8(kr[c], kr[c + NC / 2], dk, &s_w[16 * c + 8 * h]);
      f32x16 t = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c) t = mfma32(kr[c], qr[c], t);
      if (has_loc) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (p - (blk + c_row(r, h)) >= w0) s[r] = t[r];
      } else {
        s = t;
      }
    }
    after_scores();
    if (blk + kDecBlock > L) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (blk + c_row(r, h) >= L) s[r] = kNegBig;
    }
    // Online softmax for this lane's column (query head), lazily raised max.
    float mx = kNegBig;
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(s[r], s[r + 1]));
    mx = pair_max(mx);
    const bool up = mx > m_run + 8.0f;
    if (wave_any(up)) {
      const float m_new = up ? mx : m_run;
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
    }
    u32x4 pb[2];
    float ps = 0.f;
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int r = 8 * ch + 2 * w;
        const uint32_t pk = pack_bf16x2(fast_exp2(s[r] - m_run), fast_exp2(s[r + 1] - m_run));
        pb[ch][w] = pk;
        ps = sum_bf16x2(pk, ps);
      }
    l_run += ps;
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      const int key0 = 16 * ch + tr_key, key1 = key0 + 8;
      const int sw0 = swz<D>(key0), sw1 = swz<D>(key1);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = 32 * db + tr_d;
        const u32x2 v0 = read_tr(vb + key0 * D + 8 * ((d >> 3) ^ sw0) + (d & 7));
        const u32x2 v1 = read_tr(vb + key1 * D + 8 * ((d >> 3) ^ sw1) + (d & 7));
        o[db] = mfma32(u32x4{v0[0], v0[1], v1[0], v1[1]}, pb[ch], o[db]);
      }
    }
  };

  // Block i: its V tile was requested one block earlier (direct loads, double-buffered LDS); its
  // K registers were reloaded right after block i-1's score MFMAs.
  u32x4 kr[NC];
  load_k(k_begin, kr);
  load_v(k_begin, vb0);
  auto step = [&](int i, const uint16_t* vc, uint16_t* vn) __attribute__((always_inline)) {
    const int blk = k_begin + i * kDecBlock;
    const bool more = i + 1 < nblk;
    if (more) {
      load_v(blk + kDecBlock, vn);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NLD) : "memory");  // block i's K and V are in
    } else {
      wait_loads();
    }
    compute(blk, kr, vc, [&]() {
      if (more) load_k(blk + kDecBlock, kr);
    });
  };
  int i = 0;
  for (; i + 1 < nblk; i += 2) {
    step(i, vb0, vb1);
    step(i + 1, vb1, vb0);
  }
  if (i < nblk) step(i, vb0, vb1);

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

// Reduce: one workgroup of 256 threads per (query head, 32-wide slice of d, batch). Thread t
// owns splits t, t+256, ...; all of its partial loads are issued up front, then the block max of
// the split maxima, the weights exp2(m_s - M), and the weighted sums of 32 outputs are reduced
// across the 4 waves through LDS.
constexpr int kRedThreads = 256;

template <int D>
__global__ __launch_bounds__(kRedThreads) void decode_reduce_kernel(const float* __restrict__ ws, uint16_t* __restrict__ o,
                                                                    float* __restrict__ lse, int Hq, int n_splits) {
  __shared__ float s_red[kRedThreads / 64];
  __shared__ float s_acc[kRedThreads / 64][33];
  const int head = blockIdx.x, slice = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const float* src = ws + ((size_t)b * Hq + head) * n_splits * (D + 2);
  // Pass 1: maxima of this thread's splits.
  float m = kNegBig;
  for (int s = t; s < n_splits; s += kRedThreads) m = fmaxf(m, src[(size_t)s * (D + 2)]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) s_red[wave] = m;
  __syncthreads();
  float M = s_red[0];
#pragma unroll
  for (int w = 1; w < kRedThreads / 64; ++w) M = fmaxf(M, s_red[w]);
  // Pass 2: weighted sums of the denominators and of this slice's 32 outputs.
  float den = 0.f, acc[32];
#pragma unroll
  for (int d = 0; d < 32; ++d) acc[d] = 0.f;
  for (int s = t; s < n_splits; s += kRedThreads) {
    const float* ps = src + (size_t)s * (D + 2);
    const float w = fast_exp2(ps[0] - M);
    den += w * ps[1];
    const f32x4* pv = reinterpret_cast<const f32x4*>(ps + 2 + 32 * slice);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const f32x4 v = pv[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * q + e] += w * v[e];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    den += __shfl_xor(den, off);
#pragma unroll
    for (int d = 0; d < 32; ++d) acc[d] += __shfl_xor(acc[d], off);
  }
  if (lane == 0) {
#pragma unroll
    for (int d = 0; d < 32; ++d) s_acc[wave][d] = acc[d];
    s_acc[wave][32] = den;
  }
  __syncthreads();
  if (t < 32) {
    float tot = 0.f, dtot = 0.f;
#pragma unroll
    for (int w = 0; w < kRedThreads / 64; ++w) {
      tot += s_acc[w][t];
      dtot += s_acc[w][32];
    }
    o[((size_t)b * Hq + head) * D + 32 * slice + t] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(tot / dtot));
    if (lse != nullptr && slice == 0 && t == 0) lse[(size_t)b * Hq + head] = (M + __log2f(dtot)) * 0.69314718055994531f;
  }
}

DecodeSplit decode_split(long long L, int batch, int n_kv_heads) {
  // One 8-wave workgroup per CU (its V tiles use 128 KB of LDS): aim for 256 workgroups.
  const long long groups = (long long)batch * ((n_kv_heads + kDecWaves - 1) / kDecWaves);
  const long long target = (256 + groups - 1) / groups;
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
  hipLaunchKernelGGL(decode_split_kernel<D>, dim3(p.n_splits, (p.n_kv_heads + kDecWaves - 1) / kDecWaves, p.batch),
                     dim3(64 * kDecWaves), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_reduce_kernel<D>, dim3(p.n_q_heads, D / 32, p.batch), dim3(kRedThreads), 0, stream,
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
