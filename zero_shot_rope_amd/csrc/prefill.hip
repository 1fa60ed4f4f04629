// prefill.hip -- fused Dynamic Bifocal RoPE prefill attention for gfx950 (MI355X).
//
// One attention launch computes, for every query row i and query head, softmax attention over
// keys 0..i in which a pair is LOCAL when 0 <= i-j < w0 (base RoPE score q~_i . k~_j) and
// REMOTE when i-j >= w0 (score of the vectors moved to the aliased positions f(i), f(j) by the
// correction rotation Delta = f(x) - x of the post-RoPE q~, k~).
// Sources: review page "Paper Review -- Jet-Long", section Method (routing, the three
// attentions and their inclusion-exclusion merge, fusion into one kernel); gist.science
// summary, Methodologie section 2 (correction rotation by additive composition; the merge
// reaches the exact routing output with no mask matrix, stabilised by log-sum-exp).
//
// Inclusion-exclusion in registers: a local pass (pass A: base scores on pairs with
// 0 <= i-j < w0) and a remote pass (pass B minus pass C: aliased scores on pairs with
// i-j >= w0) run over the key tiles against one running max and one numerator. Each pair is
// scored in exactly one pass (the other masks it by index, no mask matrix), the two passes
// keep separate weight sums W_A and W_B - W_C, and the epilogue merges them by LSE. Nothing
// is subtracted, so there is no cancellation when W_C is close to W_B.
//
// Key correction rotation K' = R(Delta_j) K~, two modes:
//   fused       -- rotated per key tile while the tile is staged into LDS (no workspace);
//   prerotated  -- rotate_keys_kernel writes K' once per call into a caller workspace and the
//                  attention kernel stages K' tiles directly. Rotation is O(L*D) work; fused
//                  repeats it for every query tile that visits a key tile (L/BM times) inside a
//                  VALU-bound loop, so the prerotated mode is the fast one on CDNA4.
//
// Work decomposition
//   workgroup = 512 threads = 8 waves, two per SIMD, so one wave's softmax (VALU) overlaps
//   the other wave's MFMAs. One KV head, BM query positions, hpw query heads: with the 4:1
//   GQA of Qwen3-4B/8B, hpw = 4 and BM = 64, so all four heads share each staged K/V tile.
//   wave = one query head x 32 query rows (one 32-column MFMA block).
//   key tile = 64 keys. K (K~ in pass A, K' in pass R) and V are double-buffered in LDS,
//   filled by global_load_lds_dwordx4 (no registers, no VALU) into an XOR-swizzled layout;
//   tile kt-1 is in flight while tile kt is computed.
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16: each lane owns one query column, so the row max
//   and sum are in-lane plus one v_permlane32_swap; P^T feeds the PV MFMA from registers;
//   the V^T operand comes from ds_read_b64_tr_b16 on the row-major V tile; O^T accumulates
//   in 64 registers per lane. Q enters the products as given (unscaled) and the softmax scale
//   log2(e)/sqrt(D) is folded into the exponent, exp2(fma(s, scale, -m)), so the local scores
//   carry no rounding of a scaled query. The running max (log2 units) is only raised when a
//   tile's max exceeds it by more than kSlack (the output is rescaled then); otherwise
//   exponents stay <= kSlack.
//   Workgroup ids are remapped so that each of the 8 XCDs owns a contiguous range of
//   (batch, head unit, query tile) work, longest causal rows first.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace bifocal {

template <int D>
struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* krot;  // prerotated mode: K' = R(Delta) K~, same layout as k
  const uint16_t* v;
  uint16_t* o;
  float* o32;  // local-only launches: when set, O is written here in fp32 instead of bf16 to o
  float* lse;
  int B, Hq, Hkv;
  int L;       // keys 0..L-1 (the total length); query rows are the last Lq positions
  int q0, Lq;  // absolute position of query row 0 (L - Lq) and the number of query rows
  int kv_cap;  // rows per batch in k and v (the cache capacity; L for a plain prefill)
  int w0;  // clamped to [0, L]; w0 == L means every pair is local
  int G;
  int hpw;      // query heads per workgroup (1, 2 or 4)
  int n_tiles;  // query tiles per (batch, head unit)
  int n_units;  // head units per batch = Hq / hpw
  float scale_log2;
  uint32_t W[D / 2];
};

constexpr int kBN = 64;         // keys per tile
constexpr int kWaves = 8;       // waves per workgroup (two per SIMD)
constexpr int kThreads = 64 * kWaves;
// log2 units by which a row's scores may exceed the stored max before it is raised: P <= 2^64,
// row sums <= 2^81 over 2^17 keys, far inside fp32 and bf16 range, so after a row's first tile
// the max (and the rescale of O) practically never moves.
constexpr float kSlack = 64.0f;
// Scores are kept unscaled (the query enters the products as given) and the softmax scale
// log2(e)/sqrt(D) is folded into the exponent, exp2(fma(s, scale, -m)). The running max m is in
// log2 units. A half tile's raw max starts from kMaskedMax, far above the masked value kNegBig
// and far below any real score, so a fully masked half tile can only set m to kMaskedMax * scale,
// against which a masked score still has exponent below -1e28 (weight exactly 0).
constexpr float kMaskedMax = -1.0e20f;

template <int D>
struct Tile {
  static constexpr int HALF = D / 2;
  static constexpr int NC = D / 16;        // MFMA k-steps over d
  static constexpr int NDB = D / 32;       // 32-row d blocks of O^T
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;     // rows per wave-wide 1 KB direct load
  static constexpr int NLDW = kBN / RPI / kWaves;  // direct loads per wave per tile
  static constexpr int MCH = HALF / 8;     // 8-pair chunks per half row
  static constexpr int TSZ = kBN * D;      // elements per tile (rows are unpadded)
};

__device__ __forceinline__ float max3f(float a, float b, float c) { return __builtin_fmaxf(__builtin_fmaxf(a, b), c); }

// Kernel variants: every pair local (plain causal RoPE attention: w0 >= L or G = 1), or
// bifocal with the key rotation done while staging (fused) or read from a workspace.
enum PrefillMode { kLocalOnly = 0, kFused = 1, kPrerotated = 2 };

template <int D, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(const PrefillArgs<D> a) {
  using T = Tile<D>;
  constexpr int HALF = T::HALF, NC = T::NC, NDB = T::NDB, CPR = T::CPR, RPI = T::RPI, MCH = T::MCH;
  constexpr bool kBif = MODE != kLocalOnly;

  // Separate objects per buffer (not one indexed array), so the compiler can tell the tile
  // being read from the tile whose direct loads are in flight and does not wait for them.
  __shared__ __align__(16) uint16_t s_k0[T::TSZ], s_k1[T::TSZ];
  __shared__ __align__(16) uint16_t s_v0[T::TSZ], s_v1[T::TSZ];
  __shared__ uint32_t s_w[HALF];

  const int tid = threadIdx.x;
  // The wave index is uniform across the wave: from the scalar unit, everything derived from it
  // alone (the head, the wave's rows, the per-tile routing) stays scalar too.
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;

  // ---- work item: XCD-aware remap of the linear workgroup id ----
  const int nwg = gridDim.x, bid = blockIdx.x;
  const int per = nwg >> 3, rem = nwg & 7, xcd = bid & 7, slot = bid >> 3;
  const int work = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  const int tile = a.n_tiles - 1 - work % a.n_tiles;  // longest rows first
  const int bu = work / a.n_tiles;
  const int unit = bu % a.n_units, b = bu / a.n_units;
  const int Hg = a.Hq / a.Hkv;
  const int upk = Hg / a.hpw;
  const int kvh = unit / upk;
  const int head = kvh * Hg + (unit % upk) * a.hpw + (wave % a.hpw);
  const int BM = 32 * (kWaves / a.hpw);
  const int i0 = a.q0 + tile * BM;  // absolute position of the tile's first query row
  const int iw = i0 + 32 * (wave / a.hpw);  // this wave's 32 query rows
  const int L = a.L, w0 = a.w0, G = a.G;
  const float qscale = a.scale_log2;

  for (int t = tid; t < HALF; t += kThreads) s_w[t] = a.W[t];
  __syncthreads();

  const size_t q_row_stride = (size_t)a.Hq * D;
  const int qi = iw + col;  // this lane's query row
  // Query operand (B of S^T = K Q^T): lane (col, h) holds q[qi][16c + 8h .. +8] as given; with
  // `rotate`, the correction rotation R(Delta_qi) of it (in fp32, rounded once to bf16).
  auto load_q = [&](bool rotate, u32x4 (&dst)[NC]) __attribute__((always_inline)) {
    const uint16_t* src = a.q + ((size_t)b * a.Lq + (qi - a.q0)) * q_row_stride + (size_t)head * D + 8 * h;
    u32x4 raw[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      raw[c] = u32x4{0, 0, 0, 0};
      if (qi < L) raw[c] = *reinterpret_cast<const u32x4*>(src + 16 * c);
    }
    if (rotate) {
      const int dq = correction_offset(qi < L ? qi : 0, G);
#pragma unroll
      for (int c = 0; c < NC / 2; ++c) {
        u32x4 lo = raw[c], hi = raw[c + NC / 2];
        rotate8(lo, hi, dq, &s_w[16 * c + 8 * h]);
        dst[c] = lo;
        dst[c + NC / 2] = hi;
      }
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) dst[c] = raw[c];
    }
  };

  const int i_last = min(i0 + BM, L) - 1;
  const int iw_last = min(iw + 31, L - 1);
  const bool wave_live = iw <= L - 1;
  const size_t kv_row_stride = (size_t)a.Hkv * D;
  const size_t kv_off = (size_t)b * a.kv_cap * kv_row_stride + (size_t)kvh * D;
  const size_t krot_off = (size_t)b * L * kv_row_stride + (size_t)kvh * D;  // workspace K' is [B, L, Hkv, D]
  const uint16_t* kbase = a.k + kv_off;
  const uint16_t* vbase = a.v + kv_off;

  // ---- staging ----
  // Direct loads: wave w fills rows RPI*(NLDW*w + n) + lane/CPR; lane slot p = lane%CPR holds
  // global chunk p ^ swz(row). Rows past L are clamped to L-1: their scores are masked
  // (j > i) and their weights are 0.
  const int ld_row0 = RPI * T::NLDW * wave + lane / CPR;
  const int ld_slot = lane % CPR;
  // Byte offset of each of this lane's direct loads within a tile: row * row stride + its
  // swizzled chunk (loop-invariant, 32 bits). A tile entirely below L then needs no per-lane
  // address arithmetic: its base (src + j0 rows) is wave-uniform and computed on the scalar unit.
  uint32_t ld_off[T::NLDW];
#pragma unroll
  for (int n = 0; n < T::NLDW; ++n) {
    const int row = ld_row0 + RPI * n;
    ld_off[n] = (uint32_t)(row * (int)kv_row_stride + 8 * (ld_slot ^ swz<D>(row))) * 2u;
  }
  auto stage_direct = [&](const uint16_t* src, uint16_t* tile_lds, int j0) __attribute__((always_inline)) {
    if (j0 + kBN <= L) {
      const char* base = reinterpret_cast<const char*>(src + (size_t)j0 * kv_row_stride);
#pragma unroll
      for (int n = 0; n < T::NLDW; ++n)
        load_lds16(base + ld_off[n], tile_lds + (RPI * T::NLDW * wave + RPI * n) * D);
    } else {
#pragma unroll
      for (int n = 0; n < T::NLDW; ++n) {
        const int row = ld_row0 + RPI * n;
        const int j = min(j0 + row, L - 1);
        load_lds16(src + (size_t)j * kv_row_stride + 8 * (ld_slot ^ swz<D>(row)),
                   tile_lds + (RPI * T::NLDW * wave + RPI * n) * D);
      }
    }
  };
  // Fused mode: thread -> (key, 8-pair chunk) unit, rotated in registers, written swizzled.
  const int f_key = tid / MCH, f_chunk = tid % MCH;
  const bool f_unit = tid < kBN * MCH;
  auto fetch_k = [&](int j0, u32x4& lo, u32x4& hi) __attribute__((always_inline)) {
    lo = hi = u32x4{0, 0, 0, 0};
    if (f_unit) {
      const int j = min(j0 + f_key, L - 1);
      const uint16_t* src = kbase + (size_t)j * kv_row_stride + 8 * f_chunk;
      lo = *reinterpret_cast<const u32x4*>(src);
      hi = *reinterpret_cast<const u32x4*>(src + HALF);
    }
  };
  auto commit_k = [&](int j0, uint16_t* tile_lds, u32x4 lo, u32x4 hi) __attribute__((always_inline)) {
    if (f_unit) {
      rotate8(lo, hi, correction_offset(j0 + f_key, G), &s_w[8 * f_chunk]);
      uint16_t* row = tile_lds + f_key * D;
      const int sw = swz<D>(f_key);
      *reinterpret_cast<u32x4*>(row + 8 * (f_chunk ^ sw)) = lo;
      *reinterpret_cast<u32x4*>(row + 8 * ((f_chunk + MCH) ^ sw)) = hi;
    }
  };

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m_run = kNegBig;
  // The largest raw (unscaled) half-tile max that needs no rescale: a score s with
  // s * scale <= m_run + kSlack, kept in raw units so the check per half tile is one compare.
  const float inv_qscale = 1.0f / qscale;
  float m_lim = (kNegBig + kSlack) * inv_qscale;
  float l_pass[2] = {0.f, 0.f};  // [pass: 0 local (W_A), 1 remote (W_B - W_C)]

  // Operand offsets inside a tile (elements). K (A of S^T): row 32kb + col, chunk 2c + h.
  // V (A of O^T, transposed read): lanes of group g = lane/16 cover d = 32db + 16(g%2) + 0..15
  // and keys 16ch + 4h + 0..3 (+8 for elements 4..7); lane r of the group names 4 values of
  // row 16ch + 4h + r/4 (+8) at d = 32db + 16(g%2) + 4(r%4).
  const int k_sw = swz<D>(col);
  // Element offset of this lane's K operand chunk c within a half tile: row col, chunk 2c + h
  // swizzled. Kept in registers and hidden from the optimiser, so each operand read is one
  // register plus an immediate (the buffer and the half tile), with no address add per read.
  int k_off[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    k_off[c] = col * D + 8 * ((2 * c + h) ^ k_sw);
    asm volatile("" : "+v"(k_off[c]));
  }
  const int tr_r = lane & 15;
  const int tr_key = 4 * h + (tr_r >> 2);
  const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (tr_r & 3);

  // Half-tile pieces (32 keys, kb = 0 or 1 of a 64-key tile). qk: S^T = K Q^T (8 MFMAs).
  // mask: index mask of masked tiles (kept pairs: lo_rel <= i - j, and i - j < w0 in pass A).
  // exps: P^T = exp2(S^T - m) in bf16 and the lane's row sum (VALU). pv: O^T += V^T P^T
  // (8 MFMAs).
  auto qk = [&](const uint16_t* ks, int kb, const u32x4 (&qa)[NC], f32x16& s) __attribute__((always_inline)) {
    s = f32x16{};
    const uint16_t* khalf = ks + 32 * kb * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const u32x4 av = *reinterpret_cast<const u32x4*>(khalf + k_off[c]);
      s = mfma32(av, qa[c], s);
    }
  };
  auto mask = [&](f32x16& s, int j0, int kb, int lo_rel, bool local_pass) __attribute__((always_inline)) {
    // i - j = t - rc(r) with t per lane and half tile, rc(r) = 8(r/4) + r%4 a compile-time row
    // constant: each test compares a constant with one threshold.
    const int t = qi - j0 - 32 * kb - 4 * h;
    const int keep_le = t - lo_rel;  // i - j >= lo_rel  <=>  rc <= keep_le
    const int drop_le = t - w0;      // i - j <  w0      <=>  rc >  drop_le
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rc = 8 * (r >> 2) + (r & 3);
      const bool keep = (rc <= keep_le) && (!local_pass || rc > drop_le);
      if (!keep) s[r] = kNegBig;
    }
  };
  auto exps = [&](const f32x16& s, u32x4 (&pb)[2]) __attribute__((always_inline)) {
    float ps = 0.f;
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int r = 8 * ch + 2 * w;
        const uint32_t pk = pack_bf16x2(fast_exp2(__builtin_fmaf(s[r], qscale, -m_run)),
                                        fast_exp2(__builtin_fmaf(s[r + 1], qscale, -m_run)));
        pb[ch][w] = pk;
        ps = sum_bf16x2(pk, ps);
      }
    return ps;
  };
  auto pv = [&](const uint16_t* vs, int kb, const u32x4 (&pb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      const int key0 = 32 * kb + 16 * ch + tr_key, key1 = key0 + 8;
      const uint16_t* r0 = vs + key0 * D;
      const uint16_t* r1 = vs + key1 * D;
      const int sw0 = swz<D>(key0), sw1 = swz<D>(key1);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = 32 * db + tr_d;
        const u32x2 v0 = read_tr(r0 + 8 * ((d >> 3) ^ sw0) + (d & 7));
        const u32x2 v1 = read_tr(r1 + 8 * ((d >> 3) ^ sw1) + (d & 7));
        o[db] = mfma32(u32x4{v0[0], v0[1], v1[0], v1[1]}, pb[ch], o[db]);
      }
    }
  };

  // One half step in 16 slots of one MFMA each: slots 0-7 are the score MFMAs of the next half
  // tile (K rows 32*kb_k.. of ks into s_out, when DO_QK), slots 8-15 the PV MFMAs of the
  // previous half tile (P^T pb_prev, V rows 32*kb_v.. of vs, when DO_PV). Between them go the
  // softmax VALU of the current half tile (s_cur -> pb_cur, the exponentials against the stored
  // max; they need none of these MFMAs) and the LDS operand reads AHEAD slots ahead.
  // sched_barrier keeps the slot order, so the matrix unit and the VALU work side by side.
  // The rescale check closes the step.
  auto half_step = [&](auto do_qk, auto do_pv, const uint16_t* ks, int kb_k, const u32x4 (&qa)[NC], f32x16& s_out,
                       const uint16_t* vs, int kb_v, const u32x4 (&pb_prev)[2], const f32x16& s_cur,
                       u32x4 (&pb_cur)[2], bool local_pass) __attribute__((always_inline)) {
    constexpr bool DO_QK = decltype(do_qk)::value, DO_PV = decltype(do_pv)::value;
    constexpr int NS = NC + 2 * NDB;  // slots: NC score MFMAs, then 2 * NDB PV MFMAs
    const uint16_t* khalf = ks + 32 * kb_k * D;
    auto read_k = [&](int c) __attribute__((always_inline)) {
      return *reinterpret_cast<const u32x4*>(khalf + k_off[c]);
    };
    auto read_v = [&](int i) __attribute__((always_inline)) {
      const int ch = i / NDB, db = i % NDB;
      const int key0 = 32 * kb_v + 16 * ch + tr_key, key1 = key0 + 8;
      const int d = 32 * db + tr_d;
      const u32x2 v0 = read_tr(vs + key0 * D + 8 * ((d >> 3) ^ swz<D>(key0)) + (d & 7));
      const u32x2 v1 = read_tr(vs + key1 * D + 8 * ((d >> 3) ^ swz<D>(key1)) + (d & 7));
      return u32x4{v0[0], v0[1], v1[0], v1[1]};
    };
    // Operand of slot m (K chunk m for m < NC, V block m - NC after).
    auto read_op = [&](int m) __attribute__((always_inline)) {
      if (m < NC) return DO_QK ? read_k(m) : u32x4{0, 0, 0, 0};
      return DO_PV ? read_v(m - NC) : u32x4{0, 0, 0, 0};
    };
    if (DO_QK) s_out = f32x16{};
    constexpr int AHEAD = 3;  // operand reads run this many slots ahead of their MFMA
    u32x4 op[NS];
#pragma unroll
    for (int m = 0; m < AHEAD; ++m) op[m] = read_op(m);
    // The row sums accumulate straight into this pass's weight sum.
    float mxl = kMaskedMax, ps = l_pass[local_pass ? 0 : 1], e0 = 0.f, e1 = 0.f;
#pragma unroll
    for (int m = 0; m < NS; ++m) {
      __builtin_amdgcn_sched_barrier(0);
      if (m < NC) {
        if (DO_QK) s_out = mfma32(op[m], qa[m], s_out);
      } else {
        const int i = m - NC;
        if (DO_PV) o[i % NDB] = mfma32(op[m], pb_prev[i / NDB], o[i % NDB]);
      }
      if (m + AHEAD < NS) op[m + AHEAD] = read_op(m + AHEAD);
      // Softmax VALU chunks 16m/NS .. 16(m+1)/NS - 1: chunk 2p computes the exponentials of score
      // pair p, chunk 2p+1 packs them, adds them to the row sum and folds them into the max.
#pragma unroll
      for (int k = (16 * m) / NS; k < (16 * (m + 1)) / NS; ++k) {
        const int pr = k >> 1, r = 2 * pr;
        if ((k & 1) == 0) {
          e0 = fast_exp2(__builtin_fmaf(s_cur[r], qscale, -m_run));
          e1 = fast_exp2(__builtin_fmaf(s_cur[r + 1], qscale, -m_run));
        } else {
          const uint32_t pk = pack_bf16x2(e0, e1);
          // Pin the value to its slot: the compiler would otherwise sink the exponentials past
          // the rescale check (whose slow path recomputes them) and out of the MFMA slots.
          asm volatile("" ::"v"(pk));
          pb_cur[pr >> 2][pr & 3] = pk;
          ps = sum_bf16x2(pk, ps);
          mxl = max3f(mxl, s_cur[r], s_cur[r + 1]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (wave_any(mxl > m_lim)) {
      const float mx_raw = pair_max(mxl);
      const float m_new = __builtin_fmaxf(m_run, mx_raw * qscale);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      // At least the raw max just taken in, so the value that raised the max never raises it
      // again through the rounding of the division.
      m_lim = __builtin_fmaxf((m_new + kSlack) * inv_qscale, mx_raw);
      l_pass[0] *= alpha;
      l_pass[1] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      ps = l_pass[local_pass ? 0 : 1] + exps(s_cur, pb_cur);
    }
    l_pass[local_pass ? 0 : 1] = ps;
  };

  // One pass over n tiles kt = kt_first, kt_first-1, ... (tile t has keys j0(t) .. +63),
  // software-pipelined over 32-key halves inside each wave so the softmax VALU of one half runs
  // while the matrix unit works on its neighbours:
  //   half step (t,0): softmax(t,0) beside qk(t,1) [K_t] and pv(t-1,1) [V_{t-1}];
  //   barrier t; loads of K_{t+2} and V_{t+1} into the buffers of K_t and V_{t-1};
  //   half step (t,1): softmax(t,1) beside qk(t+1,0) [K_{t+1}] and pv(t,0) [V_t].
  // Every buffer a load targets was last read before the barrier that precedes the load, and the
  // loads are waited before the next barrier, a half step before the tile is read. Tiles where
  // this wave has no pair of the pass, or that need the index mask, are masked (all pairs masked
  // for the former). The first and last tiles are peeled (no pv before the first half, no qk
  // after the last), and the loop is unrolled by two so each step names its LDS buffers
  // statically.
  auto run_pass = [&](int kt_first, int n, const u32x4 (&qa)[NC], const uint16_t* ksrc, bool rotate_k,
                      bool local_pass, int lo_rel) __attribute__((always_inline)) {
    auto j0_of = [&](int t) { return (kt_first - t) * kBN; };
    // True when tile t needs the index mask for this wave (some pair masked, or none active).
    auto needs_mask = [&](int t) __attribute__((always_inline)) {
      const int j0 = j0_of(t);
      const int w_max = iw_last - j0, w_min = iw - (j0 + kBN - 1);
      const bool masked = local_pass ? !(w_min >= 0 && w_max < w0) : (w_min < w0);
      const bool active = wave_live && (local_pass ? (w_max >= 0 && w_min < w0) : (w_max >= w0));
      return masked || !active;
    };
    u32x4 flo, fhi;
    auto load_k = [&](int t, uint16_t* dst) __attribute__((always_inline)) {
      if (rotate_k) fetch_k(j0_of(t), flo, fhi);
      else stage_direct(ksrc, dst, j0_of(t));
    };
    auto finish_k = [&](int t, uint16_t* dst) __attribute__((always_inline)) {
      if (rotate_k) commit_k(j0_of(t), dst, flo, fhi);
    };
    // Prologue: K_0, K_1 and V_0 staged (V_0 into both V buffers, so the first tile's PV of a
    // "previous" half with P^T = 0 reads finite values and adds nothing); scores of half (0,0).
    load_k(0, s_k0);
    finish_k(0, s_k0);
    if (n > 1) {
      load_k(1, s_k1);
      finish_k(1, s_k1);
    }
    stage_direct(vbase, s_v0, j0_of(0));
    stage_direct(vbase, s_v1, j0_of(0));
    wait_loads();
    __syncthreads();
    f32x16 s0, s1;          // scores of the current tile's halves
    u32x4 p0[2], p1[2];     // P^T of half 0 (this tile) and half 1 (previous tile, then this)
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) p1[ch] = u32x4{0, 0, 0, 0};
    qk(s_k0, 0, qa, s0);
    const std::true_type yes{};
    // Every half step runs all three parts: the first tile's pv(-1, 1) adds P^T = 0, and the last
    // tile's qk(n, 0) reads a stale buffer into scores nobody uses.
    auto tile = [&](int t, const uint16_t* k_cur, uint16_t* k_other, const uint16_t* v_prev, uint16_t* v_cur)
                    __attribute__((always_inline)) {
      // k_cur = K_t; k_other = K_{t+1} now, refilled with K_{t+2}; v_prev = V_{t-1}, refilled with
      // V_{t+1}; v_cur = V_t.
      const bool msk = needs_mask(t);
      // half step (t, 0)
      if (msk) mask(s0, j0_of(t), 0, lo_rel, local_pass);
      half_step(yes, yes, k_cur, 1, qa, s1, v_prev, 1, p1, s0, p0, local_pass);
      if (t + 1 < n && rotate_k) finish_k(t + 1, k_other);  // fused mode: K_{t+1} rotated into LDS
      wait_loads();
      __syncthreads();
      if (t + 2 < n) load_k(t + 2, const_cast<uint16_t*>(k_cur));
      if (t + 1 < n) stage_direct(vbase, const_cast<uint16_t*>(v_prev), j0_of(t + 1));
      // half step (t, 1)
      if (msk) mask(s1, j0_of(t), 1, lo_rel, local_pass);
      half_step(yes, yes, k_other, 0, qa, s0, v_cur, 0, p0, s1, p1, local_pass);
    };
    int t = 0;
    for (; t + 1 < n; t += 2) {
      tile(t, s_k0, s_k1, s_v1, s_v0);
      tile(t + 1, s_k1, s_k0, s_v0, s_v1);
    }
    if (t < n) tile(t, s_k0, s_k1, s_v1, s_v0);
    // Drain: PV of the last half; V_{n-1} sits in buffer (n-1) % 2.
    if ((n - 1) & 1) pv(s_v1, 1, p1);
    else pv(s_v0, 1, p1);
    __syncthreads();  // the next pass's prologue refills the buffers
  };

  // ---------------- pass A: local pairs, tiles n_kt-1 down to kt_lo ----------------
  const int n_kt = i_last / kBN + 1;
  const int kt_lo = max(0, i0 - w0 + 1) / kBN;  // first tile with a local pair of this workgroup
  if (w0 > 0) {
    u32x4 qt[NC];
    load_q(false, qt);
    run_pass(n_kt - 1, n_kt - kt_lo, qt, kbase, false, true, 0);
  }

  // ---------------- pass R: remote pairs, tiles kt_hi-1 down to 0 ----------------
  if constexpr (kBif) {
    const int kt_hi = (i_last >= w0) ? (i_last - w0) / kBN + 1 : 0;  // tiles holding a remote pair
    if (kt_hi > 0) {
      u32x4 qr[NC];
      load_q(true, qr);
      if constexpr (MODE == kPrerotated) run_pass(kt_hi - 1, kt_hi, qr, a.krot + krot_off, false, false, w0);
      else run_pass(kt_hi - 1, kt_hi, qr, kbase, true, false, w0);
    }
  }

  // ---- epilogue: LSE merge of the local and remote weights, normalise, store ----
  const float w_a = pair_sum(l_pass[0]);  // local (pass A) weight, relative to 2^m
  const float w_r = pair_sum(l_pass[1]);  // remote (pass B minus pass C) weight
  const float den = w_a + w_r;
  const float inv = 1.0f / den;
  if (qi < L) {
    const size_t orow = ((size_t)b * a.Lq + (qi - a.q0)) * q_row_stride + (size_t)head * D;
    bool done = false;
    if constexpr (MODE == kLocalOnly) {
      if (a.o32 != nullptr) {
        float* dst = a.o32 + orow;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * g + 4 * h) =
                f32x4{o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
        done = true;
      }
    }
    if (!done) {
      uint16_t* dst = a.o + orow;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 out;
          out[0] = pack_bf16x2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
          out[1] = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
          *reinterpret_cast<u32x2*>(dst + 32 * db + 8 * g + 4 * h) = out;
        }
    }
    if (a.lse != nullptr && h == 0)
      a.lse[((size_t)b * a.Hq + head) * a.Lq + (qi - a.q0)] = (m_run + __log2f(den)) * 0.69314718055994531f;
  }
}

// ---------------------------------------------------------------------------------------------
// Wide-wave prefill (D = 128, four query heads per workgroup): a wave owns 48 query rows of one
// head, as three 16-column blocks of v_mfma_f32_16x16x32_bf16, so every K and V operand read from
// LDS feeds three MFMAs: 2/3 of the LDS bytes per unit of matrix work of the 32-row wave above.
// Measured at the 128K layer shape, the narrow kernel keeps the MFMA pipe 63% busy at a clock the
// power budget holds near 1.8 GHz; this one about 55% busy at 2.2 GHz, and finishes 4-5% sooner.
// The clock falls as the MFMA pipe gets busier: the lower LDS and VALU work is what buys the time.
// 8 waves = 4 heads x 2 row groups: BM = 96 query rows per workgroup. Registers do not allow the
// three-stage half step of the narrow kernel; a half step here is two phases:
//   1. softmax of this half's scores (P, exponentials against the stored max, row sums, max fold,
//      rescale check; a raised max scales O and the weight sum first);
//   2. this half's PV MFMAs, then the next half's score MFMAs.
// The two waves of a SIMD run these phases out of step (one row group does a tile's first softmax
// before the barrier), so one wave's softmax runs beside the other's MFMAs.
// With no lag between scores and PV, the keys of tile t+1 are read (its first score half) before
// the barrier of tile t+1, so K and V are triple-buffered: one barrier per tile still covers the
// direct loads, each issued a tile before the barrier that publishes it.
// 16x16x32 lane layout (A[i][k]: lane i + 16(k/8), element k%8; B[k][j]: lane j + 16(k/8); C[i][j]:
// lane j + 16(i/4), register i%4): lane (li, lg) scores keys 4lg + r of each 16-key block for query
// column li, and the PV's k order is the same permutation (element e: key 4lg + e of block 0 for
// e < 4, of block 1 for e >= 4), so P goes to the PV MFMA from the lane's own scores.
// ---------------------------------------------------------------------------------------------
constexpr int kWideCols = 48;  // query rows per wave
constexpr int kWideBM = 96;    // query rows per workgroup

// V tiles of the wide kernel: 16-byte chunk c of row r at c ^ 2(r & 7), so the transposed V^T reads
// (each 16-lane group: 4 rows x 2 adjacent chunks) of 32 lanes fall in 8 distinct 32-byte bank
// groups (no bank conflicts, measured).
__device__ __forceinline__ int vswz_wide(int row) { return 2 * (row & 7); }
// K tiles of the wide kernel: chunk c of row r at c ^ kswz(r). With the narrow kernel's swz, the K
// operand read (lane (li, lg): row li, chunk 4c + lg) had a 2-way bank conflict on every
// ds_read_b128 (measured), though 16 consecutive lanes read 16 distinct chunks; the narrow
// kernel's K read (lanes 0-31 at one chunk, 32-63 at the next) has none. Of the lane groupings
// that fit both measurements, one serves lanes whose bits 2 and 4 agree (rows differing in bits 0,
// 1, 3; chunks x and x ^ 2), another 8 lanes over half the banks (rows differing in bits 0 and 3;
// chunks x and x ^ 2). kswz permutes the row mod 16 (16 rows at one chunk stay distinct); its bit 1
// is row bit 2, constant in either group, so chunks x and x ^ 2 never meet; its bits 0, 2, 3 are
// row bits 0, 3, 1, distinct over the rows of either group.
__device__ __forceinline__ int kswz_wide(int row) {
  return (row & 1) | (((row >> 2) & 1) << 1) | (((row >> 3) & 1) << 2) | (((row >> 1) & 1) << 3);
}

// Sum over the four lanes of one 16x16 column (lanes l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float col_sum(float x) { x += __shfl_xor(x, 16); return pair_sum(x); }
__device__ __forceinline__ float col_max(float x) { x = __builtin_fmaxf(x, __shfl_xor(x, 16)); return pair_max(x); }

template <int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_wide_kernel(const PrefillArgs<128> a) {
  constexpr int D = 128, HALF = 64, CPR = 16, RPI = 4;
  constexpr int NLDW = kBN / RPI / kWaves;  // direct loads per wave per tile (2)
  constexpr bool kBif = MODE != kLocalOnly;
  // Three K and three V tile buffers (96 KB), separate objects named statically in the code, so the
  // compiler can tell a read of one from a direct load into another (it would otherwise wait for
  // every load in flight before the read).
  __shared__ __align__(16) uint16_t s_k0[kBN * D], s_k1[kBN * D], s_k2[kBN * D];
  __shared__ __align__(16) uint16_t s_v0[kBN * D], s_v1[kBN * D], s_v2[kBN * D];
  __shared__ uint32_t s_w[HALF];
  // Per lane, the byte offsets of its direct loads: K rows n = 0, 1, then V rows n = 0, 1.
  __shared__ __align__(16) uint32_t s_ldoff[kThreads * 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;

  // ---- work item: XCD-aware remap of the linear workgroup id ----
  const int nwg = gridDim.x, bid = blockIdx.x;
  const int per = nwg >> 3, rem = nwg & 7, xcd = bid & 7, slot = bid >> 3;
  const int work = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  const int tile = a.n_tiles - 1 - work % a.n_tiles;  // longest rows first
  const int bu = work / a.n_tiles;
  const int unit = bu % a.n_units, b = bu / a.n_units;
  const int Hg = a.Hq / a.Hkv;
  const int upk = Hg / 4;
  const int kvh = unit / upk;
  const int head = kvh * Hg + (unit % upk) * 4 + (wave & 3);
  const int i0 = a.q0 + tile * kWideBM;
  const int iw = i0 + kWideCols * (wave >> 2);  // this wave's 48 query rows
  const int L = a.L, w0 = a.w0, G = a.G;
  const float qscale = a.scale_log2;

  for (int t = tid; t < HALF; t += kThreads) s_w[t] = a.W[t];
  __syncthreads();

  const size_t q_row_stride = (size_t)a.Hq * D;
  // Query operand (B of S^T = K Q^T) of column block cb, k-step c: lane (li, lg) holds query row
  // iw + 16cb + li, d = 32c + 8lg .. +8, as given; with `rotate`, R(Delta_row) of it (pairs
  // (d, d + 64) are registers c and c + 2 of the same lane), in fp32, rounded once to bf16.
  auto load_q = [&](bool rotate, u32x4 (&dst)[3][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int cb = 0; cb < 3; ++cb) {
      const int qi = iw + 16 * cb + li;
      const uint16_t* src = a.q + ((size_t)b * a.Lq + (qi - a.q0)) * q_row_stride + (size_t)head * D + 8 * lg;
      u32x4 raw[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        raw[c] = u32x4{0, 0, 0, 0};
        if (qi < L) raw[c] = *reinterpret_cast<const u32x4*>(src + 32 * c);
      }
      if (rotate) {
        const int dq = correction_offset(qi < L ? qi : 0, G);
#pragma unroll
        for (int c = 0; c < 2; ++c) rotate8(raw[c], raw[c + 2], dq, &s_w[32 * c + 8 * lg]);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) dst[cb][c] = raw[c];
    }
  };

  const int iw_last = min(iw + kWideCols - 1, L - 1);
  const bool wave_live = iw <= L - 1;
  const size_t kv_row_stride = (size_t)a.Hkv * D;
  const size_t kv_off = (size_t)b * a.kv_cap * kv_row_stride + (size_t)kvh * D;
  const size_t krot_off = (size_t)b * L * kv_row_stride + (size_t)kvh * D;  // workspace K' is [B, L, Hkv, D]
  const uint16_t* kbase = a.k + kv_off;
  const uint16_t* vbase = a.v + kv_off;

  // ---- staging: as the narrow kernel, K tiles swizzled by kswz_wide, V tiles by vswz_wide ----
  const int ld_row0 = RPI * NLDW * wave + lane / CPR;
  const int ld_slot = lane % CPR;
  uint32_t ld_off_k[NLDW], ld_off_v[NLDW];
#pragma unroll
  for (int n = 0; n < NLDW; ++n) {
    const int row = ld_row0 + RPI * n;
    ld_off_k[n] = (uint32_t)(row * (int)kv_row_stride + 8 * (ld_slot ^ kswz_wide(row))) * 2u;
    ld_off_v[n] = (uint32_t)(row * (int)kv_row_stride + 8 * (ld_slot ^ vswz_wide(row))) * 2u;
  }
  *reinterpret_cast<u32x4*>(&s_ldoff[4 * tid]) = u32x4{ld_off_k[0], ld_off_k[1], ld_off_v[0], ld_off_v[1]};
  auto stage = [&](const uint16_t* src, uint16_t* tile_lds, int j0, auto is_v) __attribute__((always_inline)) {
    constexpr bool V = decltype(is_v)::value;
    if (j0 + kBN <= L) {
      const char* base = reinterpret_cast<const char*>(src + (size_t)j0 * kv_row_stride);
#pragma unroll
      for (int n = 0; n < NLDW; ++n)
        load_lds16(base + (V ? ld_off_v[n] : ld_off_k[n]), tile_lds + (RPI * NLDW * wave + RPI * n) * D);
    } else {
#pragma unroll
      for (int n = 0; n < NLDW; ++n) {
        const int row = ld_row0 + RPI * n;
        const int j = min(j0 + row, L - 1);
        const int sw = V ? vswz_wide(row) : kswz_wide(row);
        load_lds16(src + (size_t)j * kv_row_stride + 8 * (ld_slot ^ sw), tile_lds + (RPI * NLDW * wave + RPI * n) * D);
      }
    }
  };
  // In-loop loads: every tile after a pass's first one lies below row L - 1 (tiles go from the
  // highest keys down, and only the first can be partial), so no clamping. The lane offsets come
  // from the lane's own entry of an LDS table, one ds_read_b128 per use, so they hold no
  // registers across the tile loop (kept in registers they spilled, and each reload's wait held
  // one direct load behind the one before it), and the load takes the scalar base plus a 32-bit
  // lane offset. Recomputing them instead cost 9% more VALU instructions and 1-2% of the time.
  auto stage_full = [&](const uint16_t* src, uint16_t* tile_lds, int j0, auto is_v) __attribute__((always_inline)) {
    constexpr bool V = decltype(is_v)::value;
    const char* base = reinterpret_cast<const char*>(src + (size_t)j0 * kv_row_stride);
    const u32x4 offs = *reinterpret_cast<const u32x4*>(&s_ldoff[4 * tid]);
#pragma unroll
    for (int n = 0; n < NLDW; ++n) load_lds16(base + offs[(V ? 2 : 0) + n], tile_lds + (RPI * NLDW * wave + RPI * n) * D);
  };
  const std::true_type is_v{};
  const std::false_type is_k{};

  // K operand (A of S^T = K Q^T) of k-step c: key row 16kb + li of the half tile, chunk 4c + lg;
  // kswz depends on the row mod 16 only, so the 16-row block is an immediate offset.
  int k_off[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    k_off[c] = li * D + 8 * ((4 * c + lg) ^ kswz_wide(li));
    asm volatile("" : "+v"(k_off[c]));
  }
  // V^T operand (A of O^T += V^T P^T) of d block db: transposed reads of keys k0 = 4lg + li/4 and
  // k0 + 16, d = 16db + 4(li%4) .. +4. Chunk (2db + h) ^ 2(k0 & 7) = 2(db ^ (k0 & 7)) + h, so the
  // offset of block db is v_off ^ 16db (the pieces occupy disjoint bits).
  const int tr_k0 = 4 * lg + (li >> 2), tr_lo = 4 * (li & 3);
  int v_off = tr_k0 * D + 16 * (tr_k0 & 7) + 8 * (tr_lo >> 3) + (tr_lo & 7);
  asm volatile("" : "+v"(v_off));

  f32x4 o[8][3];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int cb = 0; cb < 3; ++cb) o[db][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float inv_qscale = 1.0f / qscale;
  // m_run: a column's running max in log2 units (the same in its four lanes). A half tile's raw
  // scores may reach (m_run + kSlack) / scale before the max is raised. l_run: the lane's share of
  // the column's weight sum. Both passes weigh against the one running max, so the LSE merge of
  // the local (W_A) and remote (W_B - W_C) weights is their sum: one running sum carries both.
  float m_run[3], l_run[3];
#pragma unroll
  for (int cb = 0; cb < 3; ++cb) {
    m_run[cb] = kNegBig;
    l_run[cb] = 0.f;
  }

  // Index mask of a half tile (keys j0 + 32kbh + 16kb + 4lg + r, query rows iw + 16cb + li):
  // kept iff lo_rel <= i - j, and i - j < w0 in the local pass.
  auto mask = [&](f32x4 (&s)[2][3], int j0, int kbh, int lo_rel, bool local_pass) __attribute__((always_inline)) {
    const int t0 = iw + li - j0 - 32 * kbh - 4 * lg;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int cb = 0; cb < 3; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + 16 * cb - 16 * kb - r;
          const bool keep = (t >= lo_rel) && (!local_pass || t < w0);
          if (!keep) s[kb][cb][r] = kNegBig;
        }
  };
  // Phase 1: P^T of this half (bf16) against the stored max, its row sums added to the weight sum,
  // the raw max fold and the rescale check. When some column's scores pass its limit, the column
  // maxima are raised, the weight sum scaled by alpha and this half's P^T and sums recomputed
  // against the new max; the caller scales O by alpha before this half's PV MFMAs. Returns whether
  // it rose.
  auto softmax = [&](const f32x4 (&s)[2][3], u32x4 (&p)[3], float (&alpha)[3]) __attribute__((always_inline)) {
    float ps[3], mxl[3];
#pragma unroll
    for (int cb = 0; cb < 3; ++cb) {
      ps[cb] = l_run[cb];
      mxl[cb] = kMaskedMax;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int kb = w >> 1, r = 2 * (w & 1);
        const uint32_t pk = pack_bf16x2(fast_exp2(__builtin_fmaf(s[kb][cb][r], qscale, -m_run[cb])),
                                        fast_exp2(__builtin_fmaf(s[kb][cb][r + 1], qscale, -m_run[cb])));
        p[cb][w] = pk;
        ps[cb] = sum_bf16x2(pk, ps[cb]);
        mxl[cb] = max3f(mxl[cb], s[kb][cb][r], s[kb][cb][r + 1]);
      }
    }
    const float lim0 = (m_run[0] + kSlack) * inv_qscale, lim1 = (m_run[1] + kSlack) * inv_qscale;
    const float lim2 = (m_run[2] + kSlack) * inv_qscale;
    if (!wave_any(mxl[0] > lim0 || mxl[1] > lim1 || mxl[2] > lim2)) {
#pragma unroll
      for (int cb = 0; cb < 3; ++cb) l_run[cb] = ps[cb];
      return false;
    }
#pragma unroll
    for (int cb = 0; cb < 3; ++cb) {
      const float mx_raw = col_max(mxl[cb]);
      const float m_new = __builtin_fmaxf(m_run[cb], mx_raw * qscale);
      alpha[cb] = fast_exp2(m_run[cb] - m_new);
      m_run[cb] = m_new;
      float acc = l_run[cb] * alpha[cb];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int kb = w >> 1, r = 2 * (w & 1);
        const uint32_t pk = pack_bf16x2(fast_exp2(__builtin_fmaf(s[kb][cb][r], qscale, -m_new)),
                                        fast_exp2(__builtin_fmaf(s[kb][cb][r + 1], qscale, -m_new)));
        p[cb][w] = pk;
        acc = sum_bf16x2(pk, acc);
      }
      l_run[cb] = acc;
    }
    return true;
  };
  // Phase 2 in 16 slots of three MFMAs (one per column block): slots 0-7 the PV MFMAs of this half
  // (V rows 32 hv .. of vs, d block = slot, P^T p), slots 8-15 the score MFMAs of the next half (K
  // rows 32 hk .. of ks into s; k-step = slot - 8). The LDS operand of a slot is read AHEAD slots
  // before it; sched_barrier keeps the slot order.
  auto phase2 = [&](const uint16_t* vs, int hv, const u32x4 (&p)[3], const uint16_t* ks, int hk,
                    const u32x4 (&qa)[3][4], f32x4 (&s)[2][3]) __attribute__((always_inline)) {
    const uint16_t* khalf = ks + 32 * hk * D;
    const uint16_t* vhalf = vs + 32 * hv * D;
    auto read_op = [&](int m) __attribute__((always_inline)) {
      if (m >= 8) {
        const int kb = (m - 8) >> 2, c = (m - 8) & 3;
        return *reinterpret_cast<const u32x4*>(khalf + 16 * kb * D + k_off[c]);
      }
      const uint16_t* r = vhalf + (v_off ^ (16 * m));
      const u32x2 v0 = read_tr(r), v1 = read_tr(r + 16 * D);
      return u32x4{v0[0], v0[1], v1[0], v1[1]};
    };
    constexpr int AHEAD = 4;
    u32x4 op[16];
#pragma unroll
    for (int m = 0; m < AHEAD; ++m) op[m] = read_op(m);
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      __builtin_amdgcn_sched_barrier(0);
      if (m + AHEAD < 16) op[m + AHEAD] = read_op(m + AHEAD);
      if (m < 8) {
#pragma unroll
        for (int cb = 0; cb < 3; ++cb) o[m][cb] = mfma16(op[m], p[cb], o[m][cb]);
      } else {
        const int kb = (m - 8) >> 2, c = (m - 8) & 3;
#pragma unroll
        for (int cb = 0; cb < 3; ++cb) s[kb][cb] = mfma16(op[m], qa[cb][c], c == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[kb][cb]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Score MFMAs alone (the first half of a pass).
  auto scores = [&](const uint16_t* ks, const u32x4 (&qa)[3][4], f32x4 (&s)[2][3]) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int kb = st >> 2, c = st & 3;
      const u32x4 ka = *reinterpret_cast<const u32x4*>(ks + 16 * kb * D + k_off[c]);
#pragma unroll
      for (int cb = 0; cb < 3; ++cb) s[kb][cb] = mfma16(ka, qa[cb][c], c == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[kb][cb]);
    }
  };

  // One pass over n tiles kt = kt_first, kt_first-1, ... (tile t holds keys j0(t) .. +63). Tile t:
  //   barrier t (for t > 0); loads of K_{t+2} and V_{t+1};
  //   half (t,0): mask, softmax; pv(t,0) [V_t] beside scores(t,1) [K_t];
  //   half (t,1): mask, softmax; pv(t,1) [V_t] beside scores(t+1,0) [K_{t+1}].
  // K and V tile t sit in buffers t % 3. A load issued after barrier t targets a buffer last read
  // before barrier t (K_{t-1}: scores(t-1,1); V_{t-2}: pv(t-2,1)) and is waited before barrier
  // t+1, which precedes its first read (scores(t+2,0) at the end of tile t+1; pv(t+1,0)). The loop
  // is unrolled by three so every buffer is named statically.
  auto run_pass = [&](int kt_first, int n, const u32x4 (&qa)[3][4], const uint16_t* ksrc, bool local_pass, int lo_rel)
                      __attribute__((always_inline)) {
    auto j0_of = [&](int t) { return (kt_first - t) * kBN; };
    auto needs_mask = [&](int t) __attribute__((always_inline)) {
      const int j0 = j0_of(t);
      const int w_max = iw_last - j0, w_min = iw - (j0 + kBN - 1);
      const bool masked = local_pass ? !(w_min >= 0 && w_max < w0) : (w_min < w0);
      const bool active = wave_live && (local_pass ? (w_max >= 0 && w_min < w0) : (w_max >= w0));
      return masked || !active;
    };
    stage(ksrc, s_k0, j0_of(0), is_k);
    if (n > 1) stage(ksrc, s_k1, j0_of(1), is_k);
    stage(vbase, s_v0, j0_of(0), is_v);
    wait_loads();
    __syncthreads();
    f32x4 s[2][3];
    scores(s_k0, qa, s);
    // Softmax of half (t, hh). Past the last tile (t == n) every score is masked: the scores there
    // came from a buffer no tile needs, and a fully masked half adds no weight.
    auto half = [&](int t, int hh, bool msk, u32x4 (&p)[3]) __attribute__((always_inline)) {
      if (t >= n) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int cb = 0; cb < 3; ++cb) s[kb][cb] = f32x4{kNegBig, kNegBig, kNegBig, kNegBig};
      } else if (msk) {
        mask(s, j0_of(t), hh, lo_rel, local_pass);
      }
      float alpha[3];
      if (softmax(s, p, alpha)) {
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
          for (int cb = 0; cb < 3; ++cb) o[db][cb] *= alpha[cb];
      }
    };
    // The two waves on a SIMD (waves w and w + 4: one per row group) run out of phase. The first
    // row group leads each tile with the softmax of its first half; the second does that softmax
    // at the end of the previous tile, before the barrier, so after the barrier it starts with its
    // MFMAs. From there, each wave's softmax VALU runs beside the other's MFMA phase. The softmax
    // reads no LDS, so the buffer protocol is unchanged.
    const bool lead = wave < 4;
    u32x4 p[3];
    if (!lead) half(0, 0, needs_mask(0), p);
    // kt, vt: buffers of tile t; kn, vn: of tile t+1; kf: of tile t+2.
    auto tile = [&](int t, const uint16_t* kt, const uint16_t* kn, uint16_t* kf, const uint16_t* vt, uint16_t* vn)
                    __attribute__((always_inline)) {
      if (t > 0) {
        wait_loads();
        __syncthreads();
      }
      if (t + 2 < n) stage_full(ksrc, kf, j0_of(t + 2), is_k);
      if (t + 1 < n) stage_full(vbase, vn, j0_of(t + 1), is_v);
      const bool msk = needs_mask(t);
      if (lead) half(t, 0, msk, p);
      phase2(vt, 0, p, kt, 1, qa, s);
      half(t, 1, msk, p);
      // In the last tile these scores read a buffer no tile needs and are not used; a branch
      // around them would carry O through two code paths.
      phase2(vt, 1, p, kn, 0, qa, s);
      if (!lead) half(t + 1, 0, t + 1 < n && needs_mask(t + 1), p);
    };
    for (int t = 0; t < n; t += 3) {
      tile(t, s_k0, s_k1, s_k2, s_v0, s_v1);
      if (t + 1 < n) tile(t + 1, s_k1, s_k2, s_k0, s_v1, s_v2);
      if (t + 2 < n) tile(t + 2, s_k2, s_k0, s_k1, s_v2, s_v0);
    }
    __syncthreads();  // the next pass's prologue refills the buffers
  };

  const int i_last = min(i0 + kWideBM, L) - 1;
  // Pass A: local pairs, tiles n_kt-1 down to kt_lo (base vectors). Pass R: remote pairs, tiles
  // kt_hi-1 down to 0 (rotated queries, keys rotated in the workspace). One loop body serves both.
  const int n_kt = i_last / kBN + 1;
  const int kt_lo = max(0, i0 - w0 + 1) / kBN;
  const int kt_hi = kBif ? ((i_last >= w0) ? (i_last - w0) / kBN + 1 : 0) : 0;
  u32x4 q[3][4];
  for (int pass = 0; pass < 2; ++pass) {
    const bool local_pass = pass == 0;
    const int n = local_pass ? (w0 > 0 ? n_kt - kt_lo : 0) : kt_hi;
    if (n <= 0) continue;
    load_q(!local_pass, q);
    run_pass(local_pass ? n_kt - 1 : kt_hi - 1, n, q, local_pass ? kbase : a.krot + krot_off, local_pass,
             local_pass ? 0 : w0);
  }

  // ---- epilogue: per column, LSE merge of the local and remote weights, normalise, store ----
#pragma unroll
  for (int cb = 0; cb < 3; ++cb) {
    const float den = col_sum(l_run[cb]);  // W_A + (W_B - W_C), relative to 2^m_run
    const float inv = 1.0f / den;
    const int qi = iw + 16 * cb + li;
    if (qi < L) {
      const size_t orow = ((size_t)b * a.Lq + (qi - a.q0)) * q_row_stride + (size_t)head * D + 4 * lg;
      bool done = false;
      if constexpr (MODE == kLocalOnly) {
        if (a.o32 != nullptr) {
#pragma unroll
          for (int db = 0; db < 8; ++db)
            *reinterpret_cast<f32x4*>(a.o32 + orow + 16 * db) = o[db][cb] * inv;
          done = true;
        }
      }
      if (!done) {
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          u32x2 out;
          out[0] = pack_bf16x2(o[db][cb][0] * inv, o[db][cb][1] * inv);
          out[1] = pack_bf16x2(o[db][cb][2] * inv, o[db][cb][3] * inv);
          *reinterpret_cast<u32x2*>(a.o + orow + 16 * db) = out;
        }
      }
      if (a.lse != nullptr && lg == 0)
        a.lse[((size_t)b * a.Hq + head) * a.Lq + (qi - a.q0)] = (m_run[cb] + __log2f(den)) * 0.69314718055994531f;
    }
  }
}

// K' = R(Delta_j) K~ for every key row j < L (prerotated mode): one thread per 8 rotation pairs.
// Reads k with kv_cap rows per batch, writes the compact [B, L, Hkv, D] workspace.
template <int D>
__global__ __launch_bounds__(256) void rotate_keys_kernel(const uint16_t* __restrict__ k, uint16_t* __restrict__ kr,
                                                          long long n_rows, int Hkv, int L, int kv_cap, int G,
                                                          const PrefillArgs<D> a) {
  constexpr int HALF = D / 2, MCH = HALF / 8;
  const long long u = (long long)blockIdx.x * 256 + threadIdx.x;
  if (u >= n_rows * MCH) return;
  const long long row = u / MCH;  // row = (b * L + j) * Hkv + g
  const int m = (int)(u % MCH);
  const long long bj = row / Hkv;
  const int g = (int)(row % Hkv);
  const int j = (int)(bj % L);
  const long long bb = bj / L;
  const size_t src = ((size_t)(bb * kv_cap + j) * Hkv + g) * D + 8 * m;
  const size_t dst = (size_t)row * D + 8 * m;
  u32x4 lo = *reinterpret_cast<const u32x4*>(k + src);
  u32x4 hi = *reinterpret_cast<const u32x4*>(k + src + HALF);
  uint32_t w[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = a.W[8 * m + e];
  rotate8(lo, hi, correction_offset(j, G), w);
  *reinterpret_cast<u32x4*>(kr + dst) = lo;
  *reinterpret_cast<u32x4*>(kr + dst + HALF) = hi;
}

template <int D>
static hipError_t launch_prefill_d(const PrefillLaunch& p, hipStream_t stream) {
  PrefillArgs<D> a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.krot = static_cast<const uint16_t*>(p.krot);
  a.v = static_cast<const uint16_t*>(p.v);
  a.o = static_cast<uint16_t*>(p.o);
  a.o32 = p.o32;
  a.lse = p.lse;
  a.B = p.batch;
  a.Hq = p.n_q_heads;
  a.Hkv = p.n_kv_heads;
  a.L = p.L;
  a.q0 = p.L - p.Lq;
  a.Lq = p.Lq;
  a.kv_cap = p.kv_cap;
  a.w0 = p.w0;
  a.G = p.G;
  const int Hg = p.n_q_heads / p.n_kv_heads;
  a.hpw = (Hg % 4 == 0) ? 4 : (Hg % 2 == 0) ? 2 : 1;
  const int BM = 32 * (kWaves / a.hpw);
  a.n_tiles = (p.Lq + BM - 1) / BM;
  a.n_units = p.n_q_heads / a.hpw;
  a.scale_log2 = p.scale_log2;
  for (int i = 0; i < D / 2; ++i) a.W[i] = p.W[i];
  // D = 128 with four query heads per workgroup, all local or keys rotated into the workspace: the
  // wide-wave kernel (48 query rows per wave, BM = 96), unless the grid is short and even. Query
  // rows at the end of a much longer cache give every workgroup the same long key range, and a
  // grid of few such workgroups finishes in whole rounds over the CUs: there the narrow kernel's
  // shorter workgroups round up to less time (4096 rows after 126976 keys, Qwen3-8B heads: 344
  // wide workgroups, 7.5 against 10.8 ms). A grid of 2048 or more, or rows starting no later
  // than their own count (causal work varying per tile, longest first), keeps the wide kernel.
  bool wide = false;
  if constexpr (D == 128) {
    if (a.hpw == 4 && (p.w0 >= p.L || p.local_only || p.krot != nullptr)) {
      const long long nwg_wide = (long long)p.batch * a.n_units * ((p.Lq + kWideBM - 1) / kWideBM);
      wide = (p.L - p.Lq) <= p.Lq || nwg_wide >= 2048;
    }
  }
  if (wide) a.n_tiles = (p.Lq + kWideBM - 1) / kWideBM;
  const long long nwg = (long long)p.batch * a.n_units * a.n_tiles;
  if (nwg <= 0 || nwg > 0x7fffffffLL) return hipErrorInvalidValue;
  // With every pair local (w0 == L, which the host also sets for G == 1) there is no remote
  // key: plain causal attention with no rotation at all. local_only asks for that pass alone
  // with w0 < L: plain sliding-window attention.
  if (p.w0 >= p.L || p.local_only) {
    if constexpr (D == 128) {
      if (wide) {
        hipLaunchKernelGGL((prefill_wide_kernel<kLocalOnly>), dim3((unsigned)nwg), dim3(kThreads), 0, stream, a);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((prefill_kernel<D, kLocalOnly>), dim3((unsigned)nwg), dim3(kThreads), 0, stream, a);
  } else if (p.krot != nullptr) {
    const long long rows = (long long)p.batch * p.L * p.n_kv_heads;
    const long long units = rows * (D / 16);
    hipLaunchKernelGGL(rotate_keys_kernel<D>, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream, a.k,
                       static_cast<uint16_t*>(p.krot), rows, p.n_kv_heads, p.L, p.kv_cap, p.G, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (D == 128) {
      if (wide) {
        hipLaunchKernelGGL((prefill_wide_kernel<kPrerotated>), dim3((unsigned)nwg), dim3(kThreads), 0, stream, a);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((prefill_kernel<D, kPrerotated>), dim3((unsigned)nwg), dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL((prefill_kernel<D, kFused>), dim3((unsigned)nwg), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream) {
  if (p.head_dim == 128) return launch_prefill_d<128>(p, stream);
  if (p.head_dim == 64) return launch_prefill_d<64>(p, stream);
  return hipErrorInvalidValue;
}

size_t prefill_workspace_bytes(long long batch, long long L, int n_kv_heads, int head_dim) {
  return static_cast<size_t>(batch * L * n_kv_heads * head_dim * 2);
}

}  // namespace bifocal
