// Split kernel: one workgroup of 8 waves per (key chunk, group of 8 KV heads, batch); wave w
//   owns KV head 8*blockIdx.y + w and walks the chunk in 32-key blocks. The 8 waves read the
//   same keys, so the workgroup streams each position's contiguous 2 KB of K and of V.
//   The correction angles depend only on the key position, so the workgroup computes one
//   cos/sin table per block (32 keys x D/2 frequencies) into LDS and every head's wave rotates
//   its keys with it. Score and output products run on v_mfma_f32_16x16x32_bf16: the query heads
//   of a KV head (up to 16) are its 16 columns; the usual groups of 4 to 8 waste less of 16
//   columns than of 32, and the accumulator is half as large.
//   K rows load straight into A-operand registers (two register sets, so the next block's keys
//   are in flight for a whole block); V goes global->LDS by direct loads into a per-wave
//   double-buffered swizzled tile read back transposed for O^T = V^T P^T. Local and remote
//   contributions share one running max; the wave writes the partial (max, sum, unnormalised
//   output) of its chunk to the workspace.
// Per-sequence lengths: the 32-key blocks of all sequences are laid end to end and every
//   workgroup of one grid (about one per CU) takes an equal run of them, which may cross
//   sequence boundaries: it walks its run one segment (the part of one sequence) at a time and
//   writes one partial per segment. The reduce merges each sequence's segments.
// Decode step on a raw new token: every workgroup applies base RoPE at p = L - 1 to its raw
//   query columns in registers; the workgroup whose chunk ends at L also takes the raw key and
//   value of position p, uses them for row p, and writes them into cache row p.
// Reduce kernels: merge the partials of all chunks (segments) by log-sum-exp and write bf16 o / lse.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace bifocal {

// load_lds16 with the non-temporal hint (cache policy bit 1 of the operand: nt on gfx950), for
// rows read once per launch: one pass over a cache larger than the last-level cache then reads
// from HBM faster than with the default policy.
__device__ __forceinline__ void load_lds16_nt(const void* g, uint16_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (LDS_AS void*)lds_base, 16, 0, 2);
}

template <int D>
struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  float* ws;
  // Decode step on a raw new token (NULL otherwise): q holds the raw query, k_new / v_new the raw
  // key and the value of position p = L - 1; the kernel applies base RoPE at p to the query and
  // the key, uses them for key p and writes key and value into cache row p (kc_w / vc_w).
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* kc_w;
  uint16_t* vc_w;
  const int32_t* lens;  // per-sequence lengths (device), or NULL: every sequence has length L
  int B;
  int Hq, Hkv, L, cap;  // L: the length, or with lens the maximum length
  int w0, G;            // with lens: w0 as requested, G unused (per sequence from wp)
  int wp;
  int n_splits, chunk;
  float scale_log2;
  uint32_t W[D / 2];
};

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecBlock = 32;  // keys per block

// V tiles: row-major 32 x D, 16-byte chunk c of row r stored at chunk c ^ vswz(r). A transposed
// read covers 16 rows x 32 bytes (two adjacent chunks 2m, 2m+1) per wave, 8 rows per half-wave:
// vswz permutes the chunk pairs so 8 consecutive rows land in 8 distinct 32-byte bank groups
// (D = 128: one row per 256-byte bank line; D = 64: two rows per line, split by row parity).
template <int D>
__device__ __forceinline__ int vswz(int row) {
  if constexpr (D == 128) return 2 * (row & 7);
  else return 2 * ((row >> 1) & 3);
}

// Workgroup barrier for the ds_write -> ds_read hand-over of the angle tables: waits for this
// wave's LDS operations only. __syncthreads (and a workgroup fence on LDS) would also wait for
// the direct global->LDS loads kept in flight across it. The memory clobber keeps the compiler
// from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt with only the vector-memory counter set (gfx9 encoding: vmcnt bits [3:0] and
// [15:14], expcnt [6:4] and lgkmcnt [11:8] left at their no-wait maxima). As a builtin, unlike
// inline asm, the compiler's own wait-count tracking sees it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Per-sequence lengths, flattened: sequence i contributes ceil(L_i / 32) blocks (lengths clamped
// to [1, maxL]), the blocks of all sequences are numbered end to end (sequence order, then block
// order), and workgroup w of nwg takes blocks [w * nb, (w + 1) * nb) with nb = ceil(total / nwg).
// Its run covers one or more segments (the part of one sequence inside the run); the segment of
// sequence i in workgroup w writes partial record w + i, distinct for every segment and below
// nwg + B. Every workgroup carries at most nb blocks whatever the mix of lengths.
__device__ __forceinline__ int varlen_len(const int32_t* lens, int i, int maxL) { return min(max(lens[i], 1), maxL); }
__device__ __forceinline__ int varlen_blocks(const int32_t* lens, int i, int maxL) {
  return (varlen_len(lens, i, maxL) + 31) / 32;
}

// Run by one wave: workgroup w's run. b0 = its first sequence, start = its first block within b0,
// remaining = blocks in the run (0: no work), P0 = blocks of the sequences before b0, nb = run
// length. Lane l first sums the blocks of sequences [l m, (l + 1) m), m = ceil(B / 64) (loads
// independent of each other); a scan over the lanes finds the lane holding block w * nb, whose m
// sequences are then scanned 64 at a time.
__device__ __forceinline__ void varlen_flat_plan(const int32_t* lens, int B, int maxL, int nwg, int w, int& b0,
                                                 int& start, int& remaining, long long& P0, long long& nb) {
  const int lane = threadIdx.x & 63;
  const int m = (B + 63) / 64;
  const int lo = min(lane * m, B), hi = min(lo + m, B);
  long long sum = 0;
  for (int i = lo; i < hi; ++i) sum += varlen_blocks(lens, i, maxL);
  long long incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long up = __shfl_up(incl, off);
    if (lane >= off) incl += up;
  }
  const long long total = __shfl(incl, 63);
  nb = (total + nwg - 1) / nwg;
  const long long first = (long long)w * nb;
  b0 = -1;
  start = 0;
  remaining = 0;
  P0 = 0;
  if (first >= total) return;
  remaining = (int)min(nb, total - first);
  const long long excl = incl - sum;
  const unsigned long long hit = __builtin_amdgcn_ballot_w64(first >= excl && first < incl);
  const int src = __builtin_ctzll(hit);
  const int lo_s = __shfl(lo, src), hi_s = __shfl(hi, src);
  long long base = __shfl(excl, src);
  for (int j0 = lo_s; j0 < hi_s && b0 < 0; j0 += 64) {
    const int j = j0 + lane;
    const int n = (j < hi_s) ? varlen_blocks(lens, j, maxL) : 0;
    long long inc = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long up = __shfl_up(inc, off);
      if (lane >= off) inc += up;
    }
    const long long ex = base + inc - n;
    const unsigned long long h2 = __builtin_amdgcn_ballot_w64(j < hi_s && first >= ex && first < ex + n);
    if (h2) {
      const int sj = __builtin_ctzll(h2);
      b0 = j0 + sj;
      P0 = __shfl(ex, sj);
      start = (int)(first - P0);
    }
    base += __shfl(inc, 63);
  }
}

// VAR: per-sequence lengths (flattened runs, lens != NULL); else one length, grid (split,
// KV-head group, batch).
template <int D, bool VAR>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_split_kernel(const DecodeArgs<D> a) {
  constexpr int HALF = D / 2;
  constexpr int NQC = D / 32;              // 32-wide d chunks of the score contraction
  constexpr int NKR = 2 * NQC;             // K registers (u32x4) per block: 2 key groups
  constexpr int NOB = D / 16;              // 16-row d blocks of O^T
  constexpr int CPR = D / 8, RPI = 64 / CPR;
  constexpr int VSZ = kDecBlock * D;       // elements of one wave's V tile
  constexpr int NLD = kDecBlock / RPI;     // direct loads per V tile
  constexpr int TSZ = kDecBlock * D;       // floats of one angle table: per key D/2 (cos, sin)
  constexpr int TPT = kDecBlock * HALF / kDecThreads;  // table entries per thread
  // Separate objects per buffer so reads of one do not wait for direct loads into the other.
  __shared__ __align__(16) uint16_t s_v0[kDecWaves * VSZ], s_v1[kDecWaves * VSZ];
  __shared__ __align__(16) float s_t0[TSZ], s_t1[TSZ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;  // MFMA 16x16 lane = li + 16 * lg
  // One segment: keys [k_begin, k_end) of sequence b (length L, group size G, window w0, both as
  // the host sets them for a single length); the partial of query head h goes to
  // rec + h * head_stride.
  auto segment = [&](int b, int L, int G, int w0, int k_begin, int k_end, float* rec, size_t head_stride)
                     __attribute__((always_inline)) {
  const int g = blockIdx.y * kDecWaves + wave;  // KV head of this wave
  const bool head_live = g < a.Hkv;
  const int gl = head_live ? g : 0;
  const int Hg = a.Hq / a.Hkv;
  const int p = L - 1;
  const int dq = correction_offset(p, G);

  // Query operand (B of S^T = K Q^T): column li = query head g*Hg + li (zero if li >= Hg), rows
  // d = 32c + 8lg .. +8, the bf16 query as given, for local and remote keys alike. A remote score
  // (R(Delta_p) q~) . (R(Delta_j) k~) equals q~ . R(Delta_j - Delta_p) k~ (the pair rotations
  // compose additively), so only the key is rotated, once, and the query enters the products
  // unrounded; the softmax scale is applied to the fp32 scores.
  const bool q_live = head_live && li < Hg;
  const uint16_t* qsrc = a.q + ((size_t)b * a.Hq + (size_t)gl * Hg + (q_live ? li : 0)) * D + 8 * lg;
  auto load_q = [&](u32x4 (&raw)[NQC]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < NQC; ++c) raw[c] = *reinterpret_cast<const u32x4*>(qsrc + 32 * c);
  };
  auto mask_q = [&](u32x4 (&raw)[NQC]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < NQC; ++c)
      if (!q_live) raw[c] = u32x4{0, 0, 0, 0};
  };
  // The q loads are issued first and masked after the first block's K and V loads are in
  // flight, so the first cache block does not wait for them.
  u32x4 qs[NQC];
  load_q(qs);

  const size_t row_stride = (size_t)a.Hkv * D;
  const uint16_t* kbase = a.kc + (size_t)b * a.cap * row_stride + (size_t)gl * D;
  const uint16_t* vbase = a.vc + (size_t)b * a.cap * row_stride + (size_t)gl * D;
  const int nblk = (k_end - k_begin + kDecBlock - 1) / kDecBlock;
  // LDS buffers are named statically (buffer 0/1 of V and of the angle table) and indexed with
  // one integer offset, so the compiler can tell every LDS read from the direct loads in flight
  // into the other buffer.
  auto vtile = [&](auto buf) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(buf)::value == 0) return s_v0;
    else return s_v1;
  };
  auto table = [&](auto buf) __attribute__((always_inline)) -> float* {
    if constexpr (decltype(buf)::value == 0) return s_t0;
    else return s_t1;
  };
  const int vwave = wave * VSZ;

  // K block: lane (li, lg) holds keys blk + li (registers 0..NQC-1) and blk + 16 + li
  // (NQC..2NQC-1), d = 32c + 8lg .. +8. Rows past L are clamped to L-1; their scores are masked.
  // Cache policies: each K load covers 64 bytes of 16 rows, half of each 128-byte line, and the
  // next load (c + 1) the other half, so K keeps the default policy, under which the line
  // fetched for the first half serves the second. V rows are read whole, 256 bytes per row
  // per load, once per launch: V takes the non-temporal hint, which streams from HBM faster.
  auto load_k = [&](int blk, u32x4 (&kr)[NKR]) __attribute__((always_inline)) {
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
      const int j = min(blk + 16 * kg + li, L - 1);
      const uint16_t* src = kbase + (size_t)j * row_stride + 8 * lg;
#pragma unroll
      for (int c = 0; c < NQC; ++c) kr[kg * NQC + c] = *reinterpret_cast<const u32x4*>(src + 32 * c);
    }
  };
  // V block -> this wave's LDS tile: load n fills rows RPI*n + lane/CPR, slot lane%CPR holding
  // global chunk slot ^ vswz(row).
  auto load_v = [&](int blk, auto buf) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int row = RPI * n + lane / CPR;
      const int j = min(blk + row, L - 1);
      load_lds16_nt(vbase + (size_t)j * row_stride + 8 * ((lane % CPR) ^ vswz<D>(row)),
                 vtile(buf) + (vwave + RPI * n * D));
    }
  };
  // Angle table of a block: row = key, (cos, sin) of (Delta_j - Delta_p) * omega_k at floats 2k, 2k+1, with
  // 16-byte chunk c of row r stored at chunk c ^ (r & 15) (16 rows read at one chunk hit 16
  // distinct bank groups). Thread t fills frequency t % HALF of keys t / HALF + (threads/HALF) n.
  const int t_k = tid % HALF, t_key0 = tid / HALF;
  const uint32_t t_w = a.W[t_k];
  auto fill_table = [&](int blk, auto buf) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < TPT; ++n) {
      const int key = t_key0 + (kDecThreads / HALF) * n;
      float sn, cs;
      turns_sincos(phase_turns(correction_offset(min(blk + key, L - 1), G) - dq, t_w), sn, cs);
      *reinterpret_cast<f32x2*>(table(buf) + (key * D + 4 * ((t_k >> 1) ^ (key & 15)) + 2 * (t_k & 1))) =
          f32x2{cs, sn};
    }
  };
  const bool need_table = (p - k_begin) >= w0;  // some key of this chunk is remote

  f32x4 o[NOB];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) o[ob] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig, l_run = 0.f;

  // V^T operand rows d = 16ob + li of O^T = V^T P^T: in each 16-lane group, lane r names
  // V[key + r/4][16ob + 4(r%4) .. +4] and receives V[key + e][16ob + li], e = 0..3, for the
  // group's keys 4lg .. 4lg+3 (first read) and 16 + 4lg .. (second read).
  const int tr_k0 = 4 * lg + (li >> 2), tr_k1 = tr_k0 + 16;
  const int tr_lo = 4 * (li & 3);  // d offset within the 16-row block
  const int tr_base0 = vwave + tr_k0 * D + (tr_lo & 7), tr_base1 = vwave + tr_k1 * D + (tr_lo & 7);
  const int tr_sw0 = vswz<D>(tr_k0), tr_sw1 = vswz<D>(tr_k1);

  // Keys blk .. blk+31: local iff p - j < w0 (the last w0 keys), else remote. Score register r
  // of key group kg holds key blk + 16kg + 4lg + r for query column li.
  auto compute = [&](int blk, const u32x4 (&kr)[NKR], auto buf) __attribute__((always_inline)) {
    const bool has_loc = (w0 > 0) && (p - (blk + kDecBlock - 1) < w0);
    const bool has_rem = (p - blk) >= w0;
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    if (has_loc) {
#pragma unroll
      for (int c = 0; c < NQC; ++c) {
        s[0] = mfma16(kr[c], qs[c], s[0]);
        s[1] = mfma16(kr[NQC + c], qs[c], s[1]);
      }
    }
    if (has_rem) {
      // Rotation R(Delta_j - Delta_p) of this lane's keys with the block's shared table, into
      // temporaries that feed the MFMAs directly (the loaded K registers stay read-only, so the
      // compiler never copies a register whose load may still be in flight).
      const float* tb = table(buf);
      f32x4 t[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kg = 0; kg < 2; ++kg) {
        const int row = 16 * kg + li;
#pragma unroll
        for (int c = 0; c < NQC / 2; ++c) {
          const u32x4 lo = kr[kg * NQC + c], hi = kr[kg * NQC + c + NQC / 2];
          u32x4 olo, ohi;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            // Frequencies 32c + 8lg + 2w, +1: table chunk 16c + 4lg + w holds (c0, s0, c1, s1).
            const f32x4 tc = *reinterpret_cast<const f32x4*>(tb + (row * D + 4 * ((16 * c + 4 * lg + w) ^ li)));
            const float x0 = bf16lo(lo[w]), x1 = bf16hi(lo[w]), y0 = bf16lo(hi[w]), y1 = bf16hi(hi[w]);
            olo[w] = pack_bf16x2(x0 * tc[0] - y0 * tc[1], x1 * tc[2] - y1 * tc[3]);
            ohi[w] = pack_bf16x2(x0 * tc[1] + y0 * tc[0], x1 * tc[3] + y1 * tc[2]);
          }
          t[kg] = mfma16(olo, qs[c], t[kg]);
          t[kg] = mfma16(ohi, qs[c + NQC / 2], t[kg]);
        }
      }
#pragma unroll
      for (int kg = 0; kg < 2; ++kg) {
        if (has_loc) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (p - (blk + 16 * kg + 4 * lg + r) >= w0) s[kg][r] = t[kg][r];
        } else {
          s[kg] = t[kg];
        }
      }
    }
    // Scores into log2 units (log2(e) / sqrt(D)), in fp32.
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) s[kg] *= a.scale_log2;
    if (blk + kDecBlock > k_end) {
#pragma unroll
      for (int kg = 0; kg < 2; ++kg)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (blk + 16 * kg + 4 * lg + r >= k_end) s[kg][r] = kNegBig;
    }
    // Online softmax for query column li (its 32 scores sit on lanes li, li+16, li+32, li+48),
    // lazily raised max.
    float mx = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(s[0][0], s[0][1]), __builtin_fmaxf(s[0][2], s[0][3])),
                               __builtin_fmaxf(__builtin_fmaxf(s[1][0], s[1][1]), __builtin_fmaxf(s[1][2], s[1][3])));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16));
    mx = pair_max(mx);
    const bool up = mx > m_run + 8.0f;
    if (wave_any(up)) {
      const float m_new = up ? mx : m_run;
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int ob = 0; ob < NOB; ++ob) o[ob] *= alpha;
    }
    // P^T as the B operand: lane (li, lg) element e is key 4lg + e (e < 4) or 16 + 4lg + e - 4
    // (e >= 4), exactly the keys of its score registers and of the V^T reads.
    u32x4 pb;
    float ps = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int kg = w >> 1, r = 2 * (w & 1);
      const uint32_t pk = pack_bf16x2(fast_exp2(s[kg][r] - m_run), fast_exp2(s[kg][r + 1] - m_run));
      pb[w] = pk;
      ps = sum_bf16x2(pk, ps);
    }
    l_run += ps;
    const uint16_t* vt = vtile(buf);
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
      const int ch = 2 * ob + (tr_lo >> 3);
      const u32x2 v0 = read_tr(vt + (tr_base0 + 8 * (ch ^ tr_sw0)));
      const u32x2 v1 = read_tr(vt + (tr_base1 + 8 * (ch ^ tr_sw1)));
      o[ob] = mfma16(u32x4{v0[0], v0[1], v1[0], v1[1]}, pb, o[ob]);
    }
  };

  // Step i: block i's K/V loads were issued one step earlier and its angle table filled before
  // the previous barrier. Issue block i+1's loads and fill its table (other buffers), wait for
  // block i's data, compute, barrier (table i+1 complete; table i free for block i+2).
  const std::integral_constant<int, 0> B0{};
  const std::integral_constant<int, 1> B1{};
  // Waves past the last KV head (n_kv_heads not a multiple of 8) run the same loads and math on
  // head 0's rows and discard the result: every load is then unconditional, which keeps the
  // compiler's wait counts exact.
  u32x4 ka[NKR], kb[NKR];
  load_v(k_begin, B0);
  load_k(k_begin, ka);
  wait_vmcnt<NKR + NLD>();  // q is in; block 0 stays in flight
  mask_q(qs);
  // Phase increments of this lane's pairs (frequencies 32c + 8lg + e), for the new token's RoPE:
  // read at uniform indices (scalar loads of the kernel arguments) and picked by lg, so no vector
  // load joins the in-order wait for the cache blocks in flight.
  auto pair_w = [&](int c, uint32_t (&w)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w0 = a.W[32 * c + e], w1 = a.W[32 * c + 8 + e];
      const uint32_t w2 = a.W[32 * c + 16 + e], w3 = a.W[32 * c + 24 + e];
      w[e] = lg < 2 ? (lg == 0 ? w0 : w1) : (lg == 2 ? w2 : w3);
    }
  };
  if (!VAR && a.k_new != nullptr) {
    // Raw query: base RoPE at p (the same fixed-point phase as the correction angles).
#pragma unroll
    for (int c = 0; c < NQC / 2; ++c) {
      uint32_t w[8];
      pair_w(c, w);
      u32x4 lo = qs[c], hi = qs[c + NQC / 2];
      rotate8(lo, hi, p, w);
      qs[c] = lo;
      qs[c + NQC / 2] = hi;
    }
  }
  if (need_table) fill_table(k_begin, B0);
  lds_barrier();
  // MORE: a block i+1 exists (always true except for the chunk's last block).
  auto step = [&](int i, u32x4 (&kc)[NKR], u32x4 (&kn)[NKR], auto cur, auto nxt, auto more) __attribute__((always_inline)) {
    const int blk = k_begin + i * kDecBlock;
    if constexpr (decltype(more)::value) {
      load_v(blk + kDecBlock, nxt);
      load_k(blk + kDecBlock, kn);
      if (need_table) fill_table(blk + kDecBlock, nxt);
      wait_vmcnt<NKR + NLD>();  // block i's K and V are in
    } else {
      // Decode step on a raw token: the chunk that ends at L holds key p = L - 1 in this, its last
      // block, and is the only one that reads cache row p (chunks are multiples of the block).
      // The raw key and value are loaded beside the block's last wait; after it, the key (rotated
      // by base RoPE at p) replaces the K registers of row p and the value the V tile's row p,
      // and both go to cache row p. Rows past p, which the loads clamp to row p, take the same
      // key and value, so the masked keys see exactly the data of a cache that already held them.
      const bool new_tok = !VAR && a.k_new != nullptr && k_end == L;
      const size_t new_row = ((size_t)b * a.Hkv + gl) * D;
      u32x4 kn_raw[NQC], vn_raw;
      if (new_tok) {
#pragma unroll
        for (int c = 0; c < NQC; ++c)
          kn_raw[c] = *reinterpret_cast<const u32x4*>(a.k_new + new_row + 32 * c + 8 * lg);
        vn_raw = *reinterpret_cast<const u32x4*>(a.v_new + new_row + 8 * (lane % CPR));
      }
      wait_vmcnt<0>();
      if (new_tok) {
#pragma unroll
        for (int c = 0; c < NQC / 2; ++c) {
          uint32_t w[8];
          pair_w(c, w);
          rotate8(kn_raw[c], kn_raw[c + NQC / 2], p, w);
        }
        const int r_p = p - blk;
#pragma unroll
        for (int kg = 0; kg < 2; ++kg)
#pragma unroll
          for (int c = 0; c < NQC; ++c)
            if (16 * kg + li >= r_p) kc[kg * NQC + c] = kn_raw[c];
        uint16_t* vt = vtile(cur);
#pragma unroll
        for (int n = 0; n < NLD; ++n) {
          const int row = RPI * n + lane / CPR;
          if (row >= r_p)
            *reinterpret_cast<u32x4*>(vt + (vwave + row * D + 8 * ((lane % CPR) ^ vswz<D>(row)))) = vn_raw;
        }
        if (head_live) {
          const size_t cache_row = (((size_t)b * a.cap + p) * a.Hkv + g) * D;
          if (li == (r_p & 15)) {
#pragma unroll
            for (int c = 0; c < NQC; ++c)
              *reinterpret_cast<u32x4*>(a.kc_w + cache_row + 32 * c + 8 * lg) = kn_raw[c];
          }
          if (lane < CPR) *reinterpret_cast<u32x4*>(a.vc_w + cache_row + 8 * lane) = vn_raw;
        }
      }
    }
    compute(blk, kc, cur);
    lds_barrier();
  };
  const std::true_type more_yes{};
  const std::false_type more_no{};
  int i = 0;
  for (; i + 2 < nblk; i += 2) {
    step(i, ka, kb, B0, B1, more_yes);
    step(i + 1, kb, ka, B1, B0, more_yes);
  }
  if (i + 1 < nblk) {
    step(i, ka, kb, B0, B1, more_yes);
    step(i + 1, kb, ka, B1, B0, more_no);
  } else if (i < nblk) {
    step(i, ka, kb, B0, B1, more_no);
  }

  // Column totals: the 4 lanes of query column li each summed 8 of its keys.
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot = pair_sum(l_tot);
  if (q_live) {
    const int head = g * Hg + li;
    float* dst = rec + (size_t)head * head_stride;
    if (lg == 0) {
      dst[0] = m_run;
      dst[1] = l_tot;
    }
    // O^T rows d = 16ob + 4lg + r of column li.
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[2 + 16 * ob + 4 * lg + r] = o[ob][r];
  }
  };  // segment

  if constexpr (!VAR) {
    const int b = (int)blockIdx.z, split = (int)blockIdx.x;
    const int k_begin = split * a.chunk;
    segment(b, a.L, a.G, a.w0, k_begin, min(a.L, k_begin + a.chunk),
            a.ws + ((size_t)b * a.Hq * a.n_splits + split) * (D + 2), (size_t)a.n_splits * (D + 2));
  } else {
    // Wave 0 plans this workgroup's run; the plan travels through the second angle table, which a
    // segment first writes after its first barrier, when every wave has read the plan.
    int* s_plan = reinterpret_cast<int*>(s_t1);
    if (wave == 0) {
      int b0, start, rem;
      long long P0, nb;
      varlen_flat_plan(a.lens, a.B, a.L, (int)gridDim.x, (int)blockIdx.x, b0, start, rem, P0, nb);
      if (lane == 0) {
        s_plan[0] = b0;
        s_plan[1] = start;
        s_plan[2] = rem;
        s_plan[3] = (int)(P0 & 0xffffffffLL);
        s_plan[4] = (int)(P0 >> 32);
        s_plan[5] = (int)(nb & 0xffffffffLL);
        s_plan[6] = (int)(nb >> 32);
      }
    }
    __syncthreads();
    const int w = (int)blockIdx.x;
    int b = __builtin_amdgcn_readfirstlane(s_plan[0]);
    int start = __builtin_amdgcn_readfirstlane(s_plan[1]);
    int rem = __builtin_amdgcn_readfirstlane(s_plan[2]);
    long long P = (long long)(uint32_t)__builtin_amdgcn_readfirstlane(s_plan[3]) |
                  ((long long)__builtin_amdgcn_readfirstlane(s_plan[4]) << 32);
    const long long nb = (long long)(uint32_t)__builtin_amdgcn_readfirstlane(s_plan[5]) |
                         ((long long)__builtin_amdgcn_readfirstlane(s_plan[6]) << 32);
    // Per sequence, after the nwg + B partial records: (first workgroup, number of workgroups),
    // written by the workgroup that holds the sequence's first block.
    int* info = reinterpret_cast<int*>(a.ws + (size_t)(gridDim.x + a.B) * a.Hq * (D + 2));
    while (rem > 0) {
      const int Lb = varlen_len(a.lens, b, a.L);
      const int nbk = (Lb + kDecBlock - 1) / kDecBlock;
      const int take = min(nbk - start, rem);
      if (start == 0 && blockIdx.y == 0 && tid == 0) {
        info[2 * b] = w;
        info[2 * b + 1] = (int)((P + nbk - 1) / nb - w + 1);
      }
      // G = max(1, ceil(L / w_pretrained)); w0 := L when G = 1 or w0 >= L, as for one length.
      const int Gb = (Lb - 1) / a.wp + 1;
      const int w0b = (Gb == 1 || a.w0 >= Lb) ? Lb : a.w0;
      segment(b, Lb, Gb, w0b, kDecBlock * start, min(Lb, kDecBlock * (start + take)),
              a.ws + (size_t)(w + b) * a.Hq * (D + 2), (size_t)(D + 2));
      rem -= take;
      P += nbk;
      ++b;
      start = 0;
    }
  }
}

// Reduce: one workgroup of 256 threads per (query head, 16-wide slice of d, batch). Thread
// (group g, dim c) takes dim c of splits g, g+16, g+32, ...: the 16 threads of a group read one
// split's 16 outputs as one coalesced 64-byte row and its (max, sum) as a broadcast. Up to 16
// splits per thread are loaded at once (one load round trip for up to 256 splits) and merged by
// a log-sum-exp against their common max; the 16 group results are merged the same way through
// LDS behind one barrier. (16-wide slices measured faster than 32- and 8-wide ones.)
constexpr int kRedThreads = 256;
constexpr int kRedDims = 16;  // d per workgroup
constexpr int kRedGroups = kRedThreads / kRedDims;
constexpr int kRedBatch = 16;  // splits per thread per load round

template <int D>
__global__ __launch_bounds__(kRedThreads) void decode_reduce_kernel(const float* __restrict__ ws, uint16_t* __restrict__ o,
                                                                    float* __restrict__ lse, int Hq, int n_splits) {
  __shared__ float s_m[kRedGroups], s_l[kRedGroups];
  __shared__ float s_acc[kRedGroups][kRedDims];
  const int head = blockIdx.x, slice = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int c = t % kRedDims, grp = t / kRedDims;
  // n_splits partials per (sequence, head), consecutive.
  const int n_have = n_splits;
  const float* src = ws + ((size_t)b * Hq + head) * n_splits * (D + 2);
  constexpr size_t sstride = D + 2;
  // Running (max, sum, output) of this thread's splits; absent splits weigh exp2(kNegBig - max).
  float m = kNegBig, l = 0.f, acc = 0.f;
  for (int s0 = grp; s0 < n_have; s0 += kRedGroups * kRedBatch) {
    // All loads of the batch first, then the masking of absent splits, so the batch is one
    // round trip (the compiler otherwise may wait on each load to reuse its register).
    f32x2 mls[kRedBatch];
    float os[kRedBatch];
#pragma unroll
    for (int u = 0; u < kRedBatch; ++u) {
      const float* ps = src + (size_t)min(s0 + kRedGroups * u, n_have - 1) * sstride;
      mls[u] = *reinterpret_cast<const f32x2*>(ps);  // rows are 8-byte aligned: D + 2 is even
      os[u] = ps[2 + kRedDims * slice + c];
    }
    float ms[kRedBatch], ls[kRedBatch];
#pragma unroll
    for (int u = 0; u < kRedBatch; ++u) {
      const bool live = s0 + kRedGroups * u < n_have;
      ms[u] = live ? mls[u][0] : kNegBig;
      ls[u] = live ? mls[u][1] : 0.f;
      os[u] = live ? os[u] : 0.f;
    }
    float mx = m;
#pragma unroll
    for (int u = 0; u < kRedBatch; ++u) mx = fmaxf(mx, ms[u]);
    const float a = fast_exp2(m - mx);
    acc *= a;
    l *= a;
#pragma unroll
    for (int u = 0; u < kRedBatch; ++u) {
      const float w = fast_exp2(ms[u] - mx);
      acc = __builtin_fmaf(w, os[u], acc);
      l = __builtin_fmaf(w, ls[u], l);
    }
    m = mx;
  }
  s_acc[grp][c] = acc;
  if (c == 0) {
    s_m[grp] = m;
    s_l[grp] = l;
  }
  __syncthreads();
  if (t < kRedDims) {
    float M = s_m[0];
#pragma unroll
    for (int g = 1; g < kRedGroups; ++g) M = fmaxf(M, s_m[g]);
    float tot = 0.f, den = 0.f;
#pragma unroll
    for (int g = 0; g < kRedGroups; ++g) {
      const float w = fast_exp2(s_m[g] - M);
      tot = __builtin_fmaf(w, s_acc[g][t], tot);
      den = __builtin_fmaf(w, s_l[g], den);
    }
    o[((size_t)b * Hq + head) * D + kRedDims * slice + t] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(tot / den));
    if (lse != nullptr && slice == 0 && t == 0) lse[(size_t)b * Hq + head] = (M + __log2f(den)) * 0.69314718055994531f;
  }
}

// Per-sequence-length reduce: one workgroup of 4 waves per (query head, sequence). Sequence b's
// segments sit in records first + b + s, s < n (each record holding every head), from the pair
// (first, n) its first workgroup wrote. With many sequences a run holds few of them, so the split
// parallelism is 4 (one wave each, up to kSeqBatch segments loaded at once) and every lane keeps
// D / 64 dimensions; a long sequence's segments take a few more load rounds.
constexpr int kSeqWaves = 4;
constexpr int kSeqBatch = 8;

template <int D>
__global__ __launch_bounds__(64 * kSeqWaves) void decode_reduce_seq_kernel(const float* __restrict__ ws,
                                                                           uint16_t* __restrict__ o,
                                                                           float* __restrict__ lse, int Hq,
                                                                           const int32_t* __restrict__ info) {
  constexpr int DPL = D / 64;  // dimensions per lane
  __shared__ float s_m[kSeqWaves], s_l[kSeqWaves];
  __shared__ float s_acc[kSeqWaves][D];
  const int head = blockIdx.x, b = blockIdx.y, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int first = info[2 * b], n_have = info[2 * b + 1];
  const float* src = ws + ((size_t)(first + b) * Hq + head) * (D + 2);
  const size_t sstride = (size_t)Hq * (D + 2);
  float m = kNegBig, l = 0.f, acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  for (int s0 = wv; s0 < n_have; s0 += kSeqWaves * kSeqBatch) {
    f32x2 mls[kSeqBatch];
    float os[kSeqBatch][DPL];
#pragma unroll
    for (int u = 0; u < kSeqBatch; ++u) {
      const float* ps = src + (size_t)min(s0 + kSeqWaves * u, n_have - 1) * sstride;
      mls[u] = *reinterpret_cast<const f32x2*>(ps);  // records start at even floats: D + 2 is even
      if constexpr (DPL == 2) {
        const f32x2 v = *reinterpret_cast<const f32x2*>(ps + 2 + 2 * lane);
        os[u][0] = v[0];
        os[u][1] = v[1];
      } else {
        os[u][0] = ps[2 + lane];
      }
    }
    float mx = m;
#pragma unroll
    for (int u = 0; u < kSeqBatch; ++u) {
      if (s0 + kSeqWaves * u >= n_have) mls[u] = f32x2{kNegBig, 0.f};
      mx = fmaxf(mx, mls[u][0]);
    }
    const float a = fast_exp2(m - mx);
    l *= a;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] *= a;
#pragma unroll
    for (int u = 0; u < kSeqBatch; ++u) {
      const float w = s0 + kSeqWaves * u < n_have ? fast_exp2(mls[u][0] - mx) : 0.f;
      l = __builtin_fmaf(w, mls[u][1], l);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = __builtin_fmaf(w, os[u][e], acc[e]);
    }
    m = mx;
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) s_acc[wv][DPL * lane + e] = acc[e];
  if (lane == 0) {
    s_m[wv] = m;
    s_l[wv] = l;
  }
  __syncthreads();
  if (wv == 0) {
    float M = s_m[0];
#pragma unroll
    for (int g = 1; g < kSeqWaves; ++g) M = fmaxf(M, s_m[g]);
    float den = 0.f, tot[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) tot[e] = 0.f;
#pragma unroll
    for (int g = 0; g < kSeqWaves; ++g) {
      const float w = fast_exp2(s_m[g] - M);
      den = __builtin_fmaf(w, s_l[g], den);
#pragma unroll
      for (int e = 0; e < DPL; ++e) tot[e] = __builtin_fmaf(w, s_acc[g][DPL * lane + e], tot[e]);
    }
    uint16_t* dst = o + ((size_t)b * Hq + head) * D + DPL * lane;
#pragma unroll
    for (int e = 0; e < DPL; ++e) dst[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(tot[e] / den));
    if (lse != nullptr && lane == 0) lse[(size_t)b * Hq + head] = (M + __log2f(den)) * 0.69314718055994531f;
  }
}

long long decode_varlen_slots(int batch, int n_kv_heads) {
  (void)batch;  // one grid of about one workgroup per CU, whatever the batch
  const long long groups = (n_kv_heads + kDecWaves - 1) / kDecWaves;
  return (256 + groups - 1) / groups;
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
  a.k_new = static_cast<const uint16_t*>(p.k_new);
  a.v_new = static_cast<const uint16_t*>(p.v_new);
  a.kc_w = p.k_new ? static_cast<uint16_t*>(const_cast<void*>(p.k_cache)) : nullptr;
  a.vc_w = p.k_new ? static_cast<uint16_t*>(const_cast<void*>(p.v_cache)) : nullptr;
  a.lens = p.lens;
  a.wp = p.w_pretrained;
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
  a.B = p.batch;
  const unsigned groups = (p.n_kv_heads + kDecWaves - 1) / kDecWaves;
  // Per-sequence lengths: n_splits is the number of workgroups along x (the flattened runs); the
  // workspace holds n_splits + batch partial records, then the per-sequence (first, count) pairs.
  const int32_t* info = nullptr;
  if (p.lens) {
    info = reinterpret_cast<const int32_t*>(p.workspace + (size_t)(p.n_splits + p.batch) * p.n_q_heads * (D + 2));
    hipLaunchKernelGGL((decode_split_kernel<D, true>), dim3(p.n_splits, groups, 1), dim3(kDecThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_split_kernel<D, false>), dim3(p.n_splits, groups, p.batch), dim3(kDecThreads), 0,
                       stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.lens)
    hipLaunchKernelGGL(decode_reduce_seq_kernel<D>, dim3(p.n_q_heads, p.batch), dim3(64 * kSeqWaves), 0, stream,
                       (const float*)p.workspace, static_cast<uint16_t*>(p.o), p.lse, p.n_q_heads, info);
  else
    hipLaunchKernelGGL(decode_reduce_kernel<D>, dim3(p.n_q_heads, D / kRedDims, p.batch), dim3(kRedThreads), 0, stream,
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
