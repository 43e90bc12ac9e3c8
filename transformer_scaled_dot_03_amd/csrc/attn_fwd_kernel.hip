// Fused scaled dot-product attention forward for gfx950 (MI355X).
//
//   O = softmax(scale * Q K^T) V   per (batch, head), optional causal and
//   key-padding masks ("Attention Is All You Need": overview page, section
//   "The idea: every word queries every word"; notebook chapter, sections
//   "Multi-Head Self-Attention" and "Masked Attention in the Decoder").
//
// One work-group owns 32 query rows per wave of one (b, head) (d = 128: 8
// waves, 256 rows; d = 64: 4 waves, 128 rows); wave w owns rows [32w, 32w + 32).
// The key/value sequence is streamed in tiles of 64 keys through LDS by
// direct-to-LDS buffer loads (double-buffered: the loads of the next tiles are
// in flight while the current ones are computed).  The softmax is the
// running (online) form: per row a running maximum m and sum l, with the
// output accumulator rescaled by exp2(m_old - m_new) whenever m grows
// (Milakov & Gimelshein 2018, "Online normalizer calculation for softmax";
// the pages only name the fused FlashAttention family).  The score matrix is
// never written to memory.
//
// Matrix-core mapping (bf16 path, v_mfma_f32_32x32x16_bf16, 64-lane wave,
// lane l, g = l / 32, c = l % 32):
//   * S^T = K Q^T: the A operand is a 32-key slice of K from LDS, the B
//     operand is the wave's Q rows held in registers.  The accumulator then
//     holds, in lane l, query row c and 16 of the 32 keys; lane l ^ 32 holds
//     the other 16 keys of the same row.  Row max and row sum therefore need a
//     single exchange between the two lane halves.
//   * The K rows are fed in the order sigma (bits 2 and 3 of the key slot
//     swapped), so accumulator registers 8m .. 8m+7 of a lane hold 8
//     consecutive keys 16m + 8g + (0..7).  Those 8 probabilities are exactly
//     the B operand of O^T = V^T P^T for keys 16m .. 16m+15: no data movement
//     between the two products.
//   * V stays row-major in LDS; the A operand of the second product (8 keys
//     of one output column per lane) comes from two transposing LDS reads
//     (ds_read_b64_tr_b16).
//   * Each step interleaves the matrix operations of one tile with the vector
//     work of another (P V of the previous tile with this tile's row maxima,
//     then the next tile's scores with this tile's exponentials), in a pinned
//     instruction order.
//   * The output accumulator O^T holds, in lane l, row c and d/2 contiguous
//     output columns (dv permuted by tau), so the epilogue writes d bytes of
//     contiguous bf16 per lane.
// The fp32 path uses v_mfma_f32_32x32x2_f32 with the same S^T form; its PV
// product takes one key per lane per step, so V needs no transpose there.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_device.h"
#include "attn_launch.h"

// A test-only build (-DATTN_FWD_TEST_SERIAL_STAGING=1, built as
// libattn_serial_test.so, never as libattn.so) waits for each step's K/V loads
// before the step reads LDS: no load is in flight while any wave reads a tile,
// so the staging cannot race; its outputs must equal the pipelined kernel's
// bit for bit.
#ifndef ATTN_FWD_TEST_SERIAL_STAGING
#define ATTN_FWD_TEST_SERIAL_STAGING 0
#endif

namespace attn {

constexpr bool kSerialStaging = ATTN_FWD_TEST_SERIAL_STAGING != 0;

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------

// Shape of the bf16 kernel per head size:
//   kWaves  waves per work-group;
//   kRG     groups of 32 query rows per wave: with 2, every K and V^T fragment
//           read from LDS feeds two MFMAs (half the LDS reads per flop), at
//           the price of ~400 registers (accumulators in AGPRs): one wave per SIMD;
//   kBN     keys per pipeline step (the K/V tile; K and V double-buffered);
//   kMinWaves  waves per SIMD the register budget must allow (d = 64: three
//           work-groups per CU, at most 168 registers per lane).
// Measured on MI355X for d = 128 (T = 16384): 8 waves x 1 group x 64 keys is
// fastest; two row groups (one wave per SIMD) ran ~30% slower and deeper
// prefetch (3 or 4 buffers) did not help.
template <int D>
struct Bf16Shape;
template <>
struct Bf16Shape<64> {
  static constexpr int kWaves = 4, kRG = 1, kBN = 64, kMinWaves = 3;
};
template <>
struct Bf16Shape<128> {
  static constexpr int kWaves = 8, kRG = 1, kBN = 64, kMinWaves = 2;
};

template <int D, bool CAUSAL, bool KEYPAD>
__global__ __launch_bounds__(64 * Bf16Shape<D>::kWaves, Bf16Shape<D>::kMinWaves) void attn_fwd_bf16_kernel(
    Params p) {
  constexpr int WAVES = Bf16Shape<D>::kWaves;
  constexpr int RG = Bf16Shape<D>::kRG;      // 32-row groups per wave
  constexpr int BN = Bf16Shape<D>::kBN;      // keys per tile
  constexpr int NH = BN / 32;                // 32-key slices per tile
  constexpr int BM = 32 * RG * WAVES;        // query rows per work-group
  constexpr int ROWB = D * 2;                // bytes per K / V row
  constexpr int TILEB = BN * ROWB;           // bytes per K (or V) tile
  constexpr int NLD = TILEB / 1024 / WAVES;  // 1 KB direct loads per wave per tile
  constexpr int DT = D / 16;                 // MFMA steps over d for S^T
  constexpr int NO = D / 32;                 // 32-column tiles of the output
  static_assert(RG == 1 || RG == 2, "row groups");
  static_assert(BN == 32 || BN == 64 || BN == 128, "tile keys");
  static_assert(NLD >= 1 && TILEB % (1024 * WAVES) == 0, "tile shape");
  constexpr float kNegInf = -__builtin_inff();

  // two buffers per tensor, each its own array: the compiler can then see
  // that direct-to-LDS loads into one buffer never alias reads of the other,
  // and does not wait for the prefetch before reading the current tile
  __shared__ __attribute__((aligned(1024))) char kb0[TILEB];
  __shared__ __attribute__((aligned(1024))) char kb1[TILEB];
  __shared__ __attribute__((aligned(1024))) char vb0[TILEB];
  __shared__ __attribute__((aligned(1024))) char vb1[TILEB];
  auto kbuf = [&](auto I) -> char* {
    if constexpr (decltype(I)::value % 2 == 0) return kb0;
    else return kb1;
  };
  auto vbuf = [&](auto I) -> char* {
    if constexpr (decltype(I)::value % 2 == 0) return vb0;
    else return vb1;
  };

  // ---- work-group -> unit (b, head, query tile).  The hardware hands
  // work-group ids to the 8 XCDs in turn (id % 8 is the XCD) and, within an
  // XCD, starts them in id order as earlier ones finish.  Without a mask
  // every unit is equal and each XCD gets a contiguous range of ids, so one
  // head's query tiles share its L2.  With a mask the id is read as a rank:
  //   causal: XCD x takes the heads x, x + 8, ... in groups of up to 16, and
  //     within a group the query tiles from the last (longest) down, so the
  //     short tiles fill the gaps and the tail while a group's keys and values
  //     stay in the XCD's L2 (B h not a multiple of 8: all heads form one group);
  //   key padding: (b, query tile, head), so every batch entry's lengths are
  //     spread over all XCDs (head h on XCD h % 8 when h is a multiple of 8)
  //     instead of a contiguous range of batch entries landing on one XCD.
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;
  int bh, qt;
  if (CAUSAL) {
    const int nbh = p.B * p.H;
    int qd;
    if (nbh % kXcds == 0) {
      const int per_xcd = nbh / kXcds;
      int hg = 16;                        // heads per group: a power of two dividing per_xcd
      while (per_xcd % hg != 0) hg >>= 1;
      const int x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
      const int grp = j / (hg * p.n_qtiles), k = j - grp * (hg * p.n_qtiles);
      qd = k / hg;
      bh = x + kXcds * (grp * hg + (k - qd * hg));
    } else {
      qd = blockIdx.x / nbh;
      bh = blockIdx.x - qd * nbh;
    }
    qt = p.n_qtiles - 1 - qd;
  } else if (KEYPAD) {
    const int t = blockIdx.x / p.H;
    const int head_r = blockIdx.x - t * p.H;
    const int b_r = t / p.n_qtiles;
    qt = t - b_r * p.n_qtiles;
    bh = b_r * p.H + head_r;
  } else {
    tile_of_block(p.n_qtiles, false, bh, qt);
  }

  const int b = bh / p.H;
  const int Tq = p.Tq, Tk = p.Tk;
  const int q0 = qt * BM;
  const int qw = q0 + 32 * RG * w;     // first row of this wave; group r holds rows qw + 32r + c

  int kend = Tk;                       // keys [0, kend) hold data
  if (KEYPAD) kend = min(kend, clamp_len(p.key_lens, b, Tk));
  int kend_wg = kend;
  if (CAUSAL) kend_wg = min(kend_wg, q0 + BM);
  const int ntiles = kend_wg > 0 ? (kend_wg + BN - 1) / BN : 0;
  int kend_w = CAUSAL ? min(kend, qw + 32 * RG) : kend;
  if (qw >= Tq) kend_w = 0;            // wave entirely past the last row
  const int ntw = kend_w > 0 ? (kend_w + BN - 1) / BN : 0;

  // tensors addressed through (batch, head, row) strides; rows are d contiguous elements
  const int head = bh - b * p.H;
  const __bf16* Qg = static_cast<const __bf16*>(p.q) + b * p.q_sb + head * p.q_sh;
  const __bf16* Kg = static_cast<const __bf16*>(p.k) + b * p.k_sb + head * p.k_sh;
  const __bf16* Vg = static_cast<const __bf16*>(p.v) + b * p.v_sb + head * p.v_sh;
  __bf16* Og = static_cast<__bf16*>(p.o) + b * p.o_sb + head * p.o_sh;
  const uint32_t krs = 2u * p.k_sr, vrs = 2u * p.v_sr;    // row strides in bytes

  // Q rows -> registers (B operand of S^T); d index of step t is 16t + 8g + e.
  bf16x8 qf[RG][DT];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int row = qw + 32 * r + c;
    const bool ok = row < Tq;
    const __bf16* qp = Qg + (int64_t)(ok ? row : 0) * p.q_sr + 8 * g;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      u32x4 x = ok ? *reinterpret_cast<const u32x4*>(qp + 16 * t) : u32x4{0, 0, 0, 0};
      if (p.neg) x ^= 0x80008000u;     // negative scale: use -Q and |scale| (exact)
      qf[r][t] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // ---- direct-to-LDS staging: this lane's source offsets for its NLD 1 KB blocks
  uint32_t k_src[NLD], v_src[NLD];
#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    const int pos = (WAVES * u + w) * 1024 + 16 * lane;
    const int r = pos / ROWB, pc = (pos % ROWB) / 16;
    const int key = (r & ~31) + sigma32(r & 31);
    k_src[u] = key * krs + 16 * (pc ^ k_swz<D>(r));
    v_src[u] = r * vrs + 16 * (pc ^ v_swz<D>(r));
  }
  // rows at or past kend read as zero: the range ends with the last valid row's d elements
  auto load_k = [&](int j0, char* kt) {
    const __amdgpu_buffer_rsrc_t kr =
        buffer_rsrc(Kg + (int64_t)j0 * p.k_sr, (uint32_t)(kend - j0 - 1) * krs + ROWB);
#pragma unroll
    for (int u = 0; u < NLD; ++u) lds_dma16(kr, kt + (WAVES * u + w) * 1024, k_src[u]);
  };
  auto load_v = [&](int j0, char* vt) {
    const __amdgpu_buffer_rsrc_t vr =
        buffer_rsrc(Vg + (int64_t)j0 * p.v_sr, (uint32_t)(kend - j0 - 1) * vrs + ROWB);
#pragma unroll
    for (int u = 0; u < NLD; ++u) lds_dma16(vr, vt + (WAVES * u + w) * 1024, v_src[u]);
  };

  // ---- LDS read offsets (bytes, within a tile)
  // K: lane (c, g), step t reads logical chunk 2t + g of slot row 32 hh + c
  int k_rd[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) k_rd[t] = c * ROWB + 16 * ((2 * t + g) ^ k_swz<D>(c));
  // V^T via transposed reads: in each 16-lane group G (h = G & 1, g = G >> 1)
  // source lane s reads 4 consecutive output columns of key row
  // 8g + e0 + s/4 (+ 32 hh + 16 m); output lane j then holds that column of
  // keys e0 .. e0+3 -- the A operand of O^T = V^T P^T.
  int v_rd[NO];
  {
    const int G = lane >> 4, sl = lane & 15;
    const int h = G & 1, gg = G >> 1;
    const int r = 8 * gg + (sl >> 2);
#pragma unroll
    for (int i = 0; i < NO; ++i) {
      const int lc = (D / 16) * (sl & 1) + 2 * i + h;
      v_rd[i] = r * ROWB + 16 * (lc ^ v_swz<D>(r)) + 8 * ((sl >> 1) & 1);
    }
  }

  // per-lane state of each row group: output accumulator (O^T, row c,
  // columns tau), reference maximum (scaled, log2 units), its offset (0 while
  // no key has been seen), this lane's half of the row sum
  f32x16 acc[RG][NO];
  float m_run[RG], base[RG], l_run[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
#pragma unroll
    for (int i = 0; i < NO; ++i) acc[r][i] = f32x16{};
    m_run[r] = kNegInf;
    base[r] = 0.f;
    l_run[r] = 0.f;
  }
  const float cs = p.scale_log2;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // S^T = K Q^T for the BN keys of a K tile: register e of s[r][hh] holds
  // key 32hh + 16(e/8) + 8g + e%8 of the tile for row qw + 32r + c
  auto scores = [&](const char* kt, f32x16 (&s)[RG][NH]) {
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
#pragma unroll
      for (int r = 0; r < RG; ++r) s[r][hh] = f32x16{};
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt + 32 * hh * ROWB + k_rd[t]);
#pragma unroll
        for (int r = 0; r < RG; ++r)
          s[r][hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[r][t], s[r][hh], 0, 0, 0);
      }
    }
  };

  // O^T += V^T P^T over one V tile
  auto pv = [&](const char* v_cur, const bf16x8 (&pk)[RG][NH][2]) {
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < NO; ++i) {
          const char* vb = v_cur + (32 * hh + 16 * m) * ROWB + v_rd[i];
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 4 * ROWB));
          const bf16x8 vf =
              __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int r = 0; r < RG; ++r)
            acc[r][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pk[r][hh][m], acc[r][i], 0, 0, 0);
        }
  };

  {
    // Step j: O^T += V^T P(j-1)^T on the matrix cores interleaved with the row
    // maxima of tile j on the vector ALUs; the (rare) rescale; then S(j+1) =
    // K(j+1) Q^T on the matrix cores interleaved with the exponentials of
    // tile j.  Step j reads V(j-1) and K(j+1) and loads K(j+2) and V(j).
    // A wave issues in order and an MFMA waits for the matrix pipe, so
    // without the pinned interleave the compiler's order (all MFMAs of a
    // block, then all vector work) leaves one unit idle while the other runs.
    // zero-initialised: waves whose rows all lie past Tq (ragged last query
    // tile) still run the interior steps with the rest of the work-group;
    // their results are never stored, but they compute on defined values
    f32x16 s2[2][RG][NH];
    bf16x8 pk[RG][NH][2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < RG; ++r)
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) s2[u][r][hh] = f32x16{};
#pragma unroll
    for (int r = 0; r < RG; ++r)
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) pk[r][hh][0] = pk[r][hh][1] = bf16x8{};
    float m_tile[RG];
    auto row_max = [&](int j0, f32x16 (&sc)[RG][NH], auto MASKED) -> bool {
      if (decltype(MASKED)::value && ((j0 + BN > kend) || (CAUSAL && j0 + BN - 1 > qw))) {
        // key j0 + 8g + off(e) is allowed iff off(e) < lim - j0 - 8g, lim =
        // min(kend, row + 1): one compare against a constant per score
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          int lim = kend;
          if (CAUSAL) lim = min(lim, qw + 32 * r + c + 1);
          const int rel = lim - j0 - 8 * g;
#pragma unroll
          for (int hh = 0; hh < NH; ++hh)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              sc[r][hh][e] = (32 * hh + 16 * (e >> 3) + (e & 7)) < rel ? sc[r][hh][e] : kNegInf;
        }
      }
      // IEEE maximum (NaN-propagating): gfx950's v_maximum3_f32, with no
      // canonicalising moves in front of it (a NaN score makes the row NaN
      // through its exponential either way)
      auto vmax = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
      bool grow = false;
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        float mx[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) mx[k] = sc[r][k / 2][8 * (k % 2)];
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx[(2 * hh + e / 8) % 4] = vmax(mx[(2 * hh + e / 8) % 4], sc[r][hh][e]);
        const float m4 = vmax(vmax(mx[0], mx[1]), vmax(mx[2], mx[3]));
        const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(m4), __float_as_uint(m4), false, false);
        m_tile[r] = vmax(__uint_as_float(pr[0]), __uint_as_float(pr[1])) * cs;
        grow = grow || (m_tile[r] > m_run[r] + kRescaleThreshold);
      }
      return grow;
    };
    auto rescale = [&]() {
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        const float m_new = fmaxf(m_run[r], m_tile[r]);
        const float b_new = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run[r] - b_new);
        m_run[r] = m_new;
        base[r] = b_new;
        l_run[r] *= alpha;
#pragma unroll
        for (int i = 0; i < NO; ++i) acc[r][i] *= alpha;
      }
    };
    auto probs = [&](const f32x16 (&sc)[RG][NH]) {
#pragma unroll
      for (int r = 0; r < RG; ++r)
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            f32x8 e8;
#pragma unroll
            for (int j = 0; j < 8; ++j)
              e8[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r][hh][8 * m + j], cs, -base[r]));
            pk[r][hh][m] = __builtin_convertvector(e8, bf16x8);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const bf16x2 pr2 = {pk[r][hh][m][2 * j], pk[r][hh][m][2 * j + 1]};
              l_run[r] = __builtin_amdgcn_fdot2_f32_bf16(pr2, ones, l_run[r], false);
            }
          }
    };
    constexpr int NPV = NH * 2 * NO * RG;   // P V^T operations, 2 LDS reads each
    constexpr int NS = NH * DT * RG;        // score operations, 1 LDS read each
    // block A order: 8 reads, then per operation: 1 MFMA, 2 VALU, 2 reads
    auto pin_a = [&]() {
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 2);
      static_for<0, NPV>([&](auto I) {
        constexpr int i = decltype(I)::value;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
        __builtin_amdgcn_sched_group_barrier(0x402, 2, 2);
        if constexpr (i + 4 < NPV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
      });
    };
    // block C order: 4 reads, then per operation: 1 MFMA, 7 VALU, 1 read
    auto pin_c = [&]() {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 3);
      static_for<0, NS>([&](auto I) {
        constexpr int i = decltype(I)::value;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
        __builtin_amdgcn_sched_group_barrier(0x402, 6, 3);
        if constexpr (i + 4 < NS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 3);
      });
    };
    // the probabilities and row sums stay in the step that computes them (the
    // compiler would otherwise sink them past the barrier into the next step)
    auto pin_p = [&]() {
#pragma unroll
      for (int r = 0; r < RG; ++r) {
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
          for (int m = 0; m < 2; ++m) asm volatile("" ::"v"(pk[r][hh][m]));
        asm volatile("" ::"v"(l_run[r]));
      }
    };
    // it: step index; U: it % 2 (buffer parity)
    auto step = [&](int it, auto U, auto MASKED) {
      constexpr int u = decltype(U)::value;
      f32x16 (&sc)[RG][NH] = s2[u];
      f32x16 (&sn)[RG][NH] = s2[u ^ 1];
      const int j0 = it * BN;
      if (it + 2 < ntiles) load_k(j0 + 2 * BN, kbuf(std::integral_constant<int, u>{}));
      if (it < ntiles) load_v(j0, vbuf(std::integral_constant<int, u>{}));
      // test build only: the step's loads land before any of its LDS reads
      if constexpr (kSerialStaging) pipeline_barrier<0>();
      if constexpr (!decltype(MASKED)::value) {
        pv(vbuf(std::integral_constant<int, u + 1>{}), pk);
        const bool grow = row_max(j0, sc, MASKED);
        pin_a();
        if (__builtin_amdgcn_ballot_w64(grow) != 0) rescale();
        scores(kbuf(std::integral_constant<int, u + 1>{}), sn);
        probs(sc);
        pin_c();
        pin_p();
      } else {
        if (it >= 1 && it - 1 < ntw) pv(vbuf(std::integral_constant<int, u + 1>{}), pk);
        if (it < ntw) {
          const bool grow = row_max(j0, sc, MASKED);
          if (__builtin_amdgcn_ballot_w64(grow) != 0) rescale();
          if (it + 1 < ntw) scores(kbuf(std::integral_constant<int, u + 1>{}), sn);
          probs(sc);
          pin_p();
        }
      }
      pipeline_barrier<0>();
    };

    // prologue: K(0), K(1); the scores of tile 0; K(0) consumed before step 0 reloads its buffer
    if (ntiles > 0) load_k(0, kb0);
    if (ntiles > 1) load_k(BN, kb1);
    pipeline_barrier<0>();
    if (ntw > 0) scores(kb0, s2[0]);
    pipeline_barrier<0>();
    // tiles [0, nint) hold no masked key for any row of the work-group
    int nint = kend / BN;
    if (CAUSAL) nint = min(nint, (q0 + 1) / BN);
    nint = min(nint, ntiles);
    // steps 0 .. ntiles; step 0 (no P V^T yet) and steps >= nint take the general path
    step(0, std::integral_constant<int, 0>{}, std::true_type{});
    int it0 = 1;
    for (; it0 + 1 < nint; it0 += 2) {
      step(it0, std::integral_constant<int, 1>{}, std::false_type{});
      step(it0 + 1, std::integral_constant<int, 0>{}, std::false_type{});
    }
    for (; it0 <= ntiles; it0 += 2) {
      step(it0, std::integral_constant<int, 1>{}, std::true_type{});
      if (it0 + 1 <= ntiles) step(it0 + 1, std::integral_constant<int, 0>{}, std::true_type{});
    }
  }

  // ---- epilogue: O = O / l, one rounding to bf16, D contiguous bytes per lane;
  // optionally the row's log-sum-exp: ln 2 * (base + log2 l), -inf if no key ----
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int row = qw + 32 * r + c;
    const float l_tot = pair_sum(l_run[r]);
    if (p.lse != nullptr && g == 0 && row < Tq)
      p.lse[(int64_t)bh * Tq + row] =
          l_tot > 0.f ? 0.69314718055994531f * (base[r] + __builtin_log2f(l_tot)) : kNegInf;
    if (row < Tq) {
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
      __bf16* op = Og + (int64_t)row * p.o_sr + (D / 2) * g;
#pragma unroll
      for (int i = 0; i < NO; ++i) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          f32x8 o8;
#pragma unroll
          for (int j = 0; j < 8; ++j) o8[j] = acc[r][i][8 * h2 + j] * inv;
          *reinterpret_cast<bf16x8*>(op + 16 * i + 8 * h2) = __builtin_convertvector(o8, bf16x8);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel (v_mfma_f32_32x32x2_f32; probabilities stay fp32)
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool KEYPAD>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_f32_kernel(Params p) {
  constexpr int BN = 32;
  constexpr int KSTR = D + 1;            // odd stride: the 32 key rows hit 32 banks
  constexpr int VSTR = D + 8;            // the two lane halves read rows 4 apart: offset 32 banks
  constexpr int K_ELEMS = BN * KSTR;
  constexpr int V_ELEMS = BN * VSTR;
  constexpr int BUF = K_ELEMS + V_ELEMS;
  constexpr int DH = D / 2;              // S^T steps (2 d-values per step)
  constexpr int NO = D / 32;
  constexpr int NC = BN * D / 4 / kThreads;   // 16-byte chunks per thread per tensor

  __shared__ __attribute__((aligned(16))) float smem[2 * BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, c = lane & 31;

  int bh, qt;
  tile_of_block(p.n_qtiles, CAUSAL, bh, qt);
  const int b = bh / p.H;
  const int Tq = p.Tq, Tk = p.Tk;
  const int q0 = qt * kBM;
  const int qw = q0 + 32 * w;
  const int row = qw + c;

  int kend = Tk;
  if (KEYPAD) kend = min(kend, clamp_len(p.key_lens, b, Tk));
  int kend_wg = kend;
  if (CAUSAL) kend_wg = min(kend_wg, q0 + kBM);
  const int ntiles = kend_wg > 0 ? (kend_wg + BN - 1) / BN : 0;
  int kend_w = CAUSAL ? min(kend, qw + 32) : kend;
  if (qw >= Tq) kend_w = 0;
  const int ntw = kend_w > 0 ? (kend_w + BN - 1) / BN : 0;

  const float* Qg = static_cast<const float*>(p.q) + (int64_t)bh * Tq * D;
  const float* Kg = static_cast<const float*>(p.k) + (int64_t)bh * Tk * D;
  const float* Vg = static_cast<const float*>(p.v) + (int64_t)bh * Tk * D;
  float* Og = static_cast<float*>(p.o) + (int64_t)bh * Tq * D;

  // Q: d index of step t for lane half g is t + (D/2) g -> D/2 contiguous floats
  float qf[DH];
  {
    const bool ok = row < Tq;
    const float* qp = Qg + (int64_t)(ok ? row : 0) * D + DH * g;
#pragma unroll
    for (int t4 = 0; t4 < DH / 4; ++t4) {
      f32x4 x = ok ? *reinterpret_cast<const f32x4*>(qp + 4 * t4) : f32x4{0, 0, 0, 0};
      if (p.neg) x = -x;
#pragma unroll
      for (int j = 0; j < 4; ++j) qf[4 * t4 + j] = x[j];
    }
  }

  f32x4 kreg[NC], vreg[NC];
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int ch = tid + kThreads * u;
      const int kr = ch / (D / 4), kc = ch % (D / 4);
      const int key = j0 + kr;
      const bool ok = key < kend;
      kreg[u] = ok ? *reinterpret_cast<const f32x4*>(Kg + (int64_t)key * D + 4 * kc) : f32x4{0, 0, 0, 0};
      vreg[u] = ok ? *reinterpret_cast<const f32x4*>(Vg + (int64_t)key * D + 4 * kc) : f32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
    float* Ks = smem + buf * BUF;
    float* Vs = Ks + K_ELEMS;
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int ch = tid + kThreads * u;
      const int kr = ch / (D / 4), kc = ch % (D / 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) Ks[kr * KSTR + 4 * kc + j] = kreg[u][j];
      *reinterpret_cast<f32x4*>(Vs + kr * VSTR + 4 * kc) = vreg[u];
    }
  };

  f32x16 acc[NO];
#pragma unroll
  for (int i = 0; i < NO; ++i) acc[i] = f32x16{};
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const float cs = p.scale_log2;

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    const int j0 = it * BN;
    if (it + 1 < ntiles) load_tile(j0 + BN);

    if (it < ntw) {
      const float* Ks = smem + cur * BUF;
      const float* Vs = Ks + K_ELEMS;
      // S^T: lane's accumulator register r is key 8(r/4) + 4g + r%4 of the tile
      f32x16 s = f32x16{};
#pragma unroll
      for (int t = 0; t < DH; ++t)
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[c * KSTR + t + DH * g], qf[t], s, 0, 0, 0);
      const bool need_mask = (j0 + BN > kend) || (CAUSAL && j0 + BN - 1 > qw);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + 8 * (r >> 2) + 4 * g + (r & 3);
          bool ok = key < kend;
          if (CAUSAL) ok = ok && key <= row;
          s[r] = ok ? s[r] : -__builtin_inff();
        }
      }
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = wave_max_pair(mx);
      const float m_tile = (mx == -__builtin_inff()) ? mx : mx * cs;
      const float m_new = fmaxf(m_run, m_tile);
      const float base = (m_new == -__builtin_inff()) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - base);
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < NO; ++i) acc[i] *= alpha;
      float lsum = l_run * alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = s[r];
        float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(x, cs, -base));
        if (need_mask) pr = (x == -__builtin_inff()) ? 0.f : pr;
        s[r] = pr;
        lsum += pr;
      }
      l_run = lsum;
      // O^T += V^T P^T: step t contracts key 8(t/4) + 4g + t%4, i.e. this lane's register t
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int key = 8 * (t >> 2) + 4 * g + (t & 3);
#pragma unroll
        for (int i = 0; i < NO; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * VSTR + 32 * i + c], s[t], acc[i], 0, 0, 0);
      }
    }

    if (it + 1 < ntiles) store_tile(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds columns 32i + 8a + 4g + (0..3) of row c
  if (row < Tq) {
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    float* op = Og + (int64_t)row * D;
#pragma unroll
    for (int i = 0; i < NO; ++i)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 o4;
#pragma unroll
        for (int j = 0; j < 4; ++j) o4[j] = acc[i][4 * a + j] * inv;
        *reinterpret_cast<f32x4*>(op + 32 * i + 8 * a + 4 * g) = o4;
      }
  }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
template <int D, bool C, bool P>
static const void* bf16_fn() { return reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<D, C, P>); }
template <int D, bool C, bool P>
static const void* f32_fn() { return reinterpret_cast<const void*>(&attn_fwd_f32_kernel<D, C, P>); }

template <int D>
static const void* pick(bool f32, bool causal, bool keypad) {
  if (f32) {
    if (causal) return keypad ? f32_fn<D, true, true>() : f32_fn<D, true, false>();
    return keypad ? f32_fn<D, false, true>() : f32_fn<D, false, false>();
  }
  if (causal) return keypad ? bf16_fn<D, true, true>() : bf16_fn<D, true, false>();
  return keypad ? bf16_fn<D, false, true>() : bf16_fn<D, false, false>();
}

static int threads_per_block(DType dt, int d) {
  if (dt == DType::F32) return kThreads;
  return 64 * (d == 128 ? Bf16Shape<128>::kWaves : Bf16Shape<64>::kWaves);
}

int rows_per_block(DType dt, int d) {
  if (dt == DType::F32) return kBM;
  return d == 128 ? 32 * Bf16Shape<128>::kRG * Bf16Shape<128>::kWaves
                  : 32 * Bf16Shape<64>::kRG * Bf16Shape<64>::kWaves;
}

hipError_t launch_fwd(const Params& prm, DType dt, int d, bool causal, bool keypad, hipStream_t stream) {
  const void* fn = (d == 64) ? pick<64>(dt == DType::F32, causal, keypad)
                             : pick<128>(dt == DType::F32, causal, keypad);
  Params local = prm;
  void* args[] = {&local};
  return hipLaunchKernel(fn, dim3(prm.n_wg), dim3(threads_per_block(dt, d)), args, 0, stream);
}

}  // namespace attn
