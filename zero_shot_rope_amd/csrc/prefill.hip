// prefill.hip -- fused Dynamic Bifocal RoPE prefill attention for gfx950 (MI355X).
//
// One launch computes, for every query row i and query head, softmax attention over keys
// 0..i in which a pair is LOCAL when 0 <= i-j < w0 (base RoPE score q~_i . k~_j) and REMOTE
// when i-j >= w0 (score of the vectors moved to the aliased positions f(i), f(j), obtained
// by the correction rotation Delta = f(x) - x of the post-RoPE q~, k~).
// Sources: review page "Paper Review -- Jet-Long", section Method (routing, the three
// attentions and their inclusion-exclusion merge, fusion into one kernel); gist.science
// summary, Methodologie section 2 (correction rotation by additive composition; the merge
// reaches the exact routing output with no mask matrix, stabilised by log-sum-exp).
//
// The inclusion-exclusion merge (W_A O_A + W_B O_B - W_C O_C) / (W_A + W_B - W_C) is
// realised in registers: B minus C is exactly the set of remote pairs, so the kernel
// routes each score by its index (no mask matrix) and accumulates local and remote
// contributions with a shared running max into one numerator, keeping separate per-row
// sums for the local (A) and remote (B - C) weights; the epilogue merges them by LSE.
// Nothing is ever subtracted, so there is no cancellation when W_C is close to W_B.
//
// Work decomposition
//   workgroup = 256 threads = 4 waves; one KV head, BM query positions, hpw query heads
//   (hpw = 4 for the 4:1 GQA of Qwen3-4B/8B, so all four heads share each staged K/V tile)
//   wave      = one query head x 64 query rows (two 32-column MFMA blocks)
//   key tile  = 64 keys: K~ (band tiles) and/or K' = R(Delta_j) K~ (tiles with remote pairs)
//               and V^T staged in LDS; the K' rotation is done once per tile per workgroup
//               while staging, shared by the 4 heads.
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16, so each lane owns one query column: the row max
//   and sum are in-lane plus one v_permlane32_swap; P^T feeds the PV MFMA straight from the
//   S^T registers; O^T = V^T P^T accumulates in 128 VGPRs per lane.
//   Workgroup ids are remapped so that the 8 XCDs each take a contiguous range of
//   (batch, head unit, query tile) work, longest causal rows first.
#include "device_common.hpp"
#include "launch.hpp"

namespace bifocal {

template <int D>
struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, L;
  int w0;  // clamped to [0, L]; w0 == L means every pair is local
  int G;
  int hpw;      // query heads per workgroup (1, 2 or 4)
  int n_tiles;  // query tiles per (batch, head unit)
  int n_units;  // head units per batch = Hq / hpw
  float scale_log2;
  uint32_t W[D / 2];
};

constexpr int kBN = 64;  // keys per tile

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_kernel(const PrefillArgs<D> a) {
  constexpr int HALF = D / 2;
  constexpr int NC = D / 16;   // MFMA k-steps over d
  constexpr int NDB = D / 32;  // 32-row d blocks of O^T
  constexpr int KP = D + 8;    // K tile pitch (bf16): row stride = 4 banks mod 32
  constexpr int VP = kBN + 4;  // V^T tile pitch (bf16): row stride = 2 banks mod 32
  constexpr int MCH = HALF / 8;             // 8-pair chunks per half row
  constexpr int KUNITS = kBN * MCH;         // (key, chunk) staging units per tile
  constexpr int VUNITS = (kBN / 4) * (D / 8);  // (4 keys x 8 d) transpose units per tile

  __shared__ __align__(16) uint16_t s_krem[kBN * KP];
  __shared__ __align__(16) uint16_t s_kloc[kBN * KP];
  __shared__ __align__(16) uint16_t s_vt[D * VP];
  __shared__ uint32_t s_w[HALF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;

  // ---- work item: XCD-aware remap of the linear workgroup id ----
  const int nwg = gridDim.x, bid = blockIdx.x;
  const int per = nwg >> 3, rem = nwg & 7, xcd = bid & 7, slot = bid >> 3;
  const int work = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  const int tile = a.n_tiles - 1 - work % a.n_tiles;  // longest rows first
  const int bu = work / a.n_tiles;
  const int unit = bu % a.n_units, b = bu / a.n_units;
  const int Hg = a.Hq / a.Hkv;
  const int upk = Hg / a.hpw;  // head units per KV head
  const int kvh = unit / upk;
  const int head = kvh * Hg + (unit % upk) * a.hpw + (wave % a.hpw);
  const int BM = 64 * (4 / a.hpw);
  const int i0 = tile * BM;
  const int iw = i0 + (wave / a.hpw) * 64;
  const int L = a.L, w0 = a.w0, G = a.G;

  for (int t = tid; t < HALF; t += 256) s_w[t] = a.W[t];
  __syncthreads();

  // ---- query operands (B of S^T = K Q^T): lane (col, h) holds q[i][16c + 8h .. +8] ----
  u32x4 qt[2][NC], qr[2][NC];
  const size_t q_row_stride = (size_t)a.Hq * D;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int i = iw + 32 * qb + col;
    const uint16_t* src = a.q + ((size_t)b * L + i) * q_row_stride + (size_t)head * D + 8 * h;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qt[qb][c] = u32x4{0, 0, 0, 0};
      if (i < L) qt[qb][c] = *reinterpret_cast<const u32x4*>(src + 16 * c);
    }
    const int dq = correction_offset(i < L ? i : 0, G);
#pragma unroll
    for (int c = 0; c < NC / 2; ++c) {
      u32x4 lo = qt[qb][c], hi = qt[qb][c + NC / 2];
      rotate8(lo, hi, dq, &s_w[16 * c + 8 * h]);
      qr[qb][c] = lo;
      qr[qb][c + NC / 2] = hi;
    }
  }

  // ---- per-thread staging constants ----
  const int m_chunk = tid % MCH;  // fixed because 256 is a multiple of MCH
  uint32_t wk[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) wk[e] = s_w[8 * m_chunk + e];

  f32x16 o[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db][0] = o[db][1] = f32x16{};
  float m_run[2] = {kNegBig, kNegBig};
  float l_loc[2] = {0.f, 0.f}, l_rem[2] = {0.f, 0.f};

  const int i_last = min(i0 + BM, L) - 1;
  const int n_kt = i_last / kBN + 1;
  const int iw_last = min(iw + 63, L - 1);
  const bool wave_live = iw <= L - 1;
  const size_t kv_row_stride = (size_t)a.Hkv * D;
  const uint16_t* kbase = a.k + (size_t)b * L * kv_row_stride + (size_t)kvh * D;
  const uint16_t* vbase = a.v + (size_t)b * L * kv_row_stride + (size_t)kvh * D;

  for (int kt = 0; kt < n_kt; ++kt) {
    const int j0 = kt * kBN;
    // Workgroup-level classification decides what to stage.
    const int g_max = i_last - j0, g_min = i0 - (j0 + kBN - 1);
    const bool need_loc = (w0 > 0) && (g_max >= 0) && (g_min < w0);
    const bool need_rem = g_max >= w0;

    // ---- stage K~ / K' rows (row-major) ----
#pragma unroll
    for (int rep = 0; rep < KUNITS / 256; ++rep) {
      const int u = tid + 256 * rep;
      const int key = u / MCH;
      const int j = j0 + key;
      u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
      if (j < L) {
        const uint16_t* src = kbase + (size_t)j * kv_row_stride + 8 * m_chunk;
        lo = *reinterpret_cast<const u32x4*>(src);
        hi = *reinterpret_cast<const u32x4*>(src + HALF);
      }
      uint16_t* row_l = s_kloc + key * KP + 8 * m_chunk;
      uint16_t* row_r = s_krem + key * KP + 8 * m_chunk;
      if (need_loc) {
        *reinterpret_cast<u32x4*>(row_l) = lo;
        *reinterpret_cast<u32x4*>(row_l + HALF) = hi;
      }
      if (need_rem) {
        rotate8(lo, hi, correction_offset(j, G), wk);
        *reinterpret_cast<u32x4*>(row_r) = lo;
        *reinterpret_cast<u32x4*>(row_r + HALF) = hi;
      }
    }
    // ---- stage V^T: each unit transposes 4 keys x 8 d in registers ----
    if (tid < VUNITS) {
      const int kg = tid / (D / 8), dg = tid % (D / 8);
      u32x4 row[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + 4 * kg + r;
        row[r] = u32x4{0, 0, 0, 0};
        if (j < L) row[r] = *reinterpret_cast<const u32x4*>(vbase + (size_t)j * kv_row_stride + 8 * dg);
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
    __syncthreads();

    // ---- wave-level classification ----
    const int w_max = iw_last - j0, w_min = iw - (j0 + kBN - 1);
    const bool w_live = wave_live && w_max >= 0;
    if (w_live) {
      const bool w_loc = (w0 > 0) && (w_min < w0);
      const bool w_rem = w_max >= w0;
      const bool all_rem = w_min >= w0;
      const bool all_loc = (w_min >= 0) && (w_max < w0);
      f32x16 s[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb][0] = s[kb][1] = f32x16{};

      const uint16_t* kfirst = w_rem ? s_krem : s_kloc;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const u32x4 av = *reinterpret_cast<const u32x4*>(kfirst + (32 * kb + col) * KP + 16 * c + 8 * h);
          if (w_rem) {
            s[kb][0] = mfma32(av, qr[0][c], s[kb][0]);
            s[kb][1] = mfma32(av, qr[1][c], s[kb][1]);
          } else {
            s[kb][0] = mfma32(av, qt[0][c], s[kb][0]);
            s[kb][1] = mfma32(av, qt[1][c], s[kb][1]);
          }
        }

      // Band tile holding both kinds of pair: add the base scores and route by index.
      if (w_loc && w_rem) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            f32x16 t = f32x16{};
#pragma unroll
            for (int c = 0; c < NC; ++c) {
              const u32x4 av = *reinterpret_cast<const u32x4*>(s_kloc + (32 * kb + col) * KP + 16 * c + 8 * h);
              t = mfma32(av, qt[qb][c], t);
            }
            const int i = iw + 32 * qb + col;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int rel = i - (j0 + 32 * kb + c_row(r, h));
              if (rel < w0) s[kb][qb][r] = t[r];
            }
          }
      }

      // ---- online softmax (scores in log2 units), local and remote sums kept apart ----
      u32x4 pb[2][2][2];  // [qb][kb][chunk]
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int i = iw + 32 * qb + col;
        float mx = kNegBig;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = s[kb][qb][r] * a.scale_log2;
            if (!(all_rem || all_loc)) {
              const int rel = i - (j0 + 32 * kb + c_row(r, h));
              if (rel < 0) x = kNegBig;
            }
            s[kb][qb][r] = x;
            mx = fmaxf(mx, x);
          }
        mx = pair_max(mx);
        const float m_new = fmaxf(m_run[qb], mx);
        const float alpha = fast_exp2(m_run[qb] - m_new);
        m_run[qb] = m_new;
        l_loc[qb] *= alpha;
        l_rem[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db][qb] *= alpha;
        float sl = 0.f, sr = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = fast_exp2(s[kb][qb][r] - m_new);
            s[kb][qb][r] = pv;
            if (all_rem) {
              sr += pv;
            } else if (all_loc) {
              sl += pv;
            } else {
              const int rel = i - (j0 + 32 * kb + c_row(r, h));
              if (rel >= w0) sr += pv; else sl += pv;
            }
          }
#pragma unroll
          for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int w = 0; w < 4; ++w)
              pb[qb][kb][ch][w] = pack_bf16x2(s[kb][qb][8 * ch + 2 * w], s[kb][qb][8 * ch + 2 * w + 1]);
        }
        l_loc[qb] += sl;
        l_rem[qb] += sr;
      }

      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int ch = 0; ch < 2; ++ch) {
            const uint16_t* vr = s_vt + (32 * db + col) * VP + 32 * kb + 16 * ch + 4 * h;
            const u32x2 v0 = *reinterpret_cast<const u32x2*>(vr);
            const u32x2 v1 = *reinterpret_cast<const u32x2*>(vr + 8);
            const u32x4 av = {v0[0], v0[1], v1[0], v1[1]};
            o[db][0] = mfma32(av, pb[0][kb][ch], o[db][0]);
            o[db][1] = mfma32(av, pb[1][kb][ch], o[db][1]);
          }
    }
    __syncthreads();
  }

  // ---- epilogue: LSE merge of the local and remote weights, normalise, store ----
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int i = iw + 32 * qb + col;
    const float w_a = pair_sum(l_loc[qb]);  // local (pass A) weight, relative to 2^m
    const float w_r = pair_sum(l_rem[qb]);  // remote (pass B minus pass C) weight
    const float den = w_a + w_r;
    const float inv = 1.0f / den;
    if (i < L) {
      uint16_t* dst = a.o + ((size_t)b * L + i) * q_row_stride + (size_t)head * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 out;
          out[0] = pack_bf16x2(o[db][qb][4 * g] * inv, o[db][qb][4 * g + 1] * inv);
          out[1] = pack_bf16x2(o[db][qb][4 * g + 2] * inv, o[db][qb][4 * g + 3] * inv);
          *reinterpret_cast<u32x2*>(dst + 32 * db + 8 * g + 4 * h) = out;
        }
      if (a.lse != nullptr && h == 0)
        a.lse[((size_t)b * a.Hq + head) * L + i] = (m_run[qb] + __log2f(den)) * 0.69314718055994531f;
    }
  }
}

template <int D>
static hipError_t launch_prefill_d(const PrefillLaunch& p, hipStream_t stream) {
  PrefillArgs<D> a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.o = static_cast<uint16_t*>(p.o);
  a.lse = p.lse;
  a.B = p.batch;
  a.Hq = p.n_q_heads;
  a.Hkv = p.n_kv_heads;
  a.L = p.L;
  a.w0 = p.w0;
  a.G = p.G;
  const int Hg = p.n_q_heads / p.n_kv_heads;
  a.hpw = (Hg % 4 == 0) ? 4 : (Hg % 2 == 0) ? 2 : 1;
  const int BM = 64 * (4 / a.hpw);
  a.n_tiles = (p.L + BM - 1) / BM;
  a.n_units = p.n_q_heads / a.hpw;
  a.scale_log2 = p.scale_log2;
  for (int i = 0; i < D / 2; ++i) a.W[i] = p.W[i];
  const long long nwg = (long long)p.batch * a.n_units * a.n_tiles;
  if (nwg <= 0 || nwg > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_kernel<D>, dim3((unsigned)nwg), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream) {
  if (p.head_dim == 128) return launch_prefill_d<128>(p, stream);
  if (p.head_dim == 64) return launch_prefill_d<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace bifocal
